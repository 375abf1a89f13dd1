// Status strings and ABI version of the indexer library.
#include "dsi.h"

extern "C" const char* dsi_status_string(int status) {
  switch (status) {
    case DSI_OK:
      return "ok";
    case DSI_EINVAL:
      return "invalid argument (null pointer, negative size, or leading dimension / stride too small)";
    case DSI_EUNSUPPORTED:
      return "unsupported parameter (outside what the kernels support)";
    case DSI_EALIGN:
      return "misaligned pointer or byte stride";
    case DSI_ELAUNCH:
      return "HIP kernel launch failed";
    case DSI_EWORKSPACE:
      return "workspace missing or too small";
    default:
      return "unknown status";
  }
}

extern "C" int dsi_abi_version(void) { return 7; }
