"""Binding of libdsi_ceiling.so: the on-device ceilings (register-only MFMA loops, HBM streaming read) and the
plain copy that calibrates HBM byte counters.  Used by the benchmark, never by the indexer path."""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsi_ceiling.so")
THREADS = 256
# kinds: f16 16x16x32, FP8 16x16x128, f16 32x32x16 on constant operands; 3 and 4 = kinds 0 and 2 on random FP8 codes
FLOP_PER_INSTR = {0: 16 * 16 * 32 * 2, 1: 16 * 16 * 128 * 2, 2: 32 * 32 * 16 * 2, 3: 16 * 16 * 32 * 2,
                  4: 32 * 32 * 16 * 2}
CHAINS = {0: 16, 1: 16, 2: 8, 3: 16, 4: 8}

_p, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_SIGNATURES = {
    "dsic_mfma_loop": (ctypes.c_int, [_i32, _i32, _i32, _p, _p]),
    "dsic_stream_read": (ctypes.c_int, [_p, _sz, _i32, _i32, _p, _p]),
    "dsic_copy": (ctypes.c_int, [_p, _p, _sz, _i32, _p]),
    "dsic_paged_read": (ctypes.c_int, [_p, ctypes.c_int64, ctypes.c_int64, _p, _i32, _i32, _i32, _i32, _i32, _p, _p]),
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


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def mfma_loop(kind: int, workgroups: int, iters: int, sink: torch.Tensor) -> int:
    """Enqueue the register-only loop; returns its flop count."""
    assert sink.dtype == torch.float32 and sink.numel() >= workgroups * THREADS and sink.is_contiguous()
    _check(lib().dsic_mfma_loop(kind, workgroups, iters, sink.data_ptr(), _stream(sink)), "dsic_mfma_loop")
    return workgroups * 4 * iters * CHAINS[kind] * FLOP_PER_INSTR[kind]


def stream_read(src: torch.Tensor, workgroups: int, sink: torch.Tensor, nontemporal: bool = False) -> int:
    """Enqueue a streaming read of all of `src` (with the non-temporal load hint if asked); returns the byte
    count."""
    assert src.is_contiguous() and sink.dtype == torch.int32 and sink.numel() >= workgroups * THREADS
    nbytes = src.numel() * src.element_size()
    _check(lib().dsic_stream_read(src.data_ptr(), nbytes, workgroups, int(nontemporal), sink.data_ptr(),
                                  _stream(src)), "dsic_stream_read")
    return nbytes


def copy(src: torch.Tensor, dst: torch.Tensor, workgroups: int) -> int:
    """Enqueue a copy of all of `src` into `dst`; returns the byte count copied."""
    nbytes = src.numel() * src.element_size()
    assert src.is_contiguous() and dst.is_contiguous() and dst.numel() * dst.element_size() >= nbytes
    _check(lib().dsic_copy(src.data_ptr(), dst.data_ptr(), nbytes, workgroups, _stream(src)), "dsic_copy")
    return nbytes


def paged_read(pool: torch.Tensor, block_stride: int, pages: torch.Tensor, page_bytes: int, workgroups: int,
               sink: torch.Tensor, pages_per_round: int = 4, nontemporal: bool = False) -> int:
    """Enqueue a read of the pages `pages` (int32 ids into `pool`; ids whose page is not in the pool are read as
    nothing, on the device: no host synchronisation); returns the byte count of the pages' reads."""
    assert pool.is_contiguous() and pages.dtype == torch.int32 and pages.is_contiguous()
    assert sink.dtype == torch.int32 and sink.numel() >= workgroups * THREADS
    _check(lib().dsic_paged_read(pool.data_ptr(), pool.numel() * pool.element_size(), block_stride, pages.data_ptr(),
                                 pages.numel(), page_bytes, pages_per_round, int(nontemporal), workgroups,
                                 sink.data_ptr(), _stream(pool)), "dsic_paged_read")
    return pages.numel() * page_bytes
