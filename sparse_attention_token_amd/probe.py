"""Binding of libdsi_probe.so: whole-range runs of the device converters the indexer kernels use, for the tests
that compare them with the CPU oracle.  Never used by the indexer path."""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsi_probe.so")

_p, _i64, _u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
_SIGNATURES = {
    "dsip_e4m3_encode_changes": (ctypes.c_int, [_u32, _i64, _p, _u32, _p, _p, _p]),
    "dsip_e4m3_decode_all": (ctypes.c_int, [_p, _p, _p]),
    "dsip_fp4_decode_all": (ctypes.c_int, [_p, _p]),
}
ENTRY_POINTS = tuple(_SIGNATURES)
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype, fn.argtypes = res, args
        _lib = h
    return _lib


def _check(code, name):
    if code != 0:
        raise RuntimeError(f"{name}: status {code}")


def _stream():
    return torch.cuda.current_stream().cuda_stream


def e4m3_encode_changes(u0, n, cap=4096):
    """(first code, [(pattern, code), ...] sorted by pattern) of the hardware E4M3 encoder over patterns
    u0 .. u0+n-1."""
    trans = torch.zeros((cap, 2), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    first = torch.zeros(1, dtype=torch.int32, device="cuda")
    _check(lib().dsip_e4m3_encode_changes(u0, n, trans.data_ptr(), cap, cnt.data_ptr(), first.data_ptr(),
                                          _stream()), "dsip_e4m3_encode_changes")
    m = int(cnt.item())
    if m > cap:
        raise RuntimeError(f"{m} changes, more than the {cap} kept")
    t = trans[:m].cpu().numpy().view("uint32")
    order = t[:, 0].argsort()
    return int(first.item()), [(int(a), int(b)) for a, b in t[order]]


def e4m3_decode_all():
    f16 = torch.zeros(256, dtype=torch.int16, device="cuda")
    bf16 = torch.zeros(256, dtype=torch.int16, device="cuda")
    _check(lib().dsip_e4m3_decode_all(f16.data_ptr(), bf16.data_ptr(), _stream()), "dsip_e4m3_decode_all")
    return f16.cpu().numpy().view("uint16"), bf16.cpu().numpy().view("uint16")


def fp4_decode_all():
    out = torch.zeros((256, 16), dtype=torch.int16, device="cuda")
    _check(lib().dsip_fp4_decode_all(out.data_ptr(), _stream()), "dsip_fp4_decode_all")
    return out.cpu().numpy().view("uint16")
