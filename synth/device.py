"""Device-side fills of the seeded synthetic inputs (synth/libsynth.so).

Bit-identical to the host definitions in ``synth``: the same stream key, the
same index, the same float32 scale, the same bf16 rounding.  Used to place
large random-init weights and pre-filled cache states directly in HBM.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_int64, c_uint32, c_uint64, c_void_p

import synth

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_fill_normal4.restype = c_int
        L.synth_fill_normal4.argtypes = [c_void_p, c_int] + [c_int64] * 8 + [c_uint64, c_uint64, c_float, c_int, c_void_p]
        L.synth_fill_uniform_int.restype = c_int
        L.synth_fill_uniform_int.argtypes = [c_void_p, c_int64, c_uint64, c_uint64, c_uint32, c_void_p]
        _lib = L
    return _lib


def fill_normal4(ptr: int, bf16: bool, dims, strides, seed: int, tid: int, std: float = 1.0,
                 start: int = 0, absval: bool = False, stream: int = 0) -> None:
    """Logical tensor ``dims`` (4 ints) drawn from stream (seed, tid), element
    index ((i0*n1+i1)*n2+i2)*n3+i3 + start, written at sum(i_k * strides[k])."""
    n0, n1, n2, n3 = [int(x) for x in dims]
    s0, s1, s2, s3 = [int(x) for x in strides]
    r = lib().synth_fill_normal4(c_void_p(ptr), 1 if bf16 else 0, n0, n1, n2, n3, s0, s1, s2, s3,
                                 synth.stream_key(seed, tid), start, float(synth.normal_scale(std)),
                                 1 if absval else 0, c_void_p(stream))
    if r != 0:
        raise RuntimeError(f"synth_fill_normal4 failed ({r})")


def fill_tensor_normal(t, seed: int, tid: int, std: float = 1.0, start: int = 0, absval: bool = False) -> None:
    """Fill a contiguous torch CUDA tensor (float32 or bfloat16) in place."""
    import torch
    assert t.is_contiguous() and t.dtype in (torch.float32, torch.bfloat16)
    fill_normal4(t.data_ptr(), t.dtype == torch.bfloat16, (1, 1, 1, t.numel()), (0, 0, 0, 1), seed, tid, std,
                 start, absval, torch.cuda.current_stream(t.device).cuda_stream)


def fill_tensor_uniform_int(t, seed: int, tid: int, n: int, start: int = 0) -> None:
    import torch
    assert t.is_contiguous() and t.dtype == torch.int32
    r = lib().synth_fill_uniform_int(c_void_p(t.data_ptr()), t.numel(), synth.stream_key(seed, tid), start, n,
                                     c_void_p(torch.cuda.current_stream(t.device).cuda_stream))
    if r != 0:
        raise RuntimeError(f"synth_fill_uniform_int failed ({r})")
