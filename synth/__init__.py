"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module holds no arithmetic of the looped decoder. It only defines how the
random-init weights, token ids and pre-filled cache states are drawn, so that
the oracle (host, NumPy) and the GPU library (device fill kernels in
``synth/csrc/synth_fill.hip``) see bit-identical inputs without either side
importing the other.

Generator (counter based, so any slice can be produced on its own):

* SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014; the 64-bit finaliser as published by
  S. Vigna).  Tensor ``(seed, tid)`` gets the stream key
  ``mix64((seed << 32) | tid)`` and its element ``i`` is the (i+1)-th output of
  SplitMix64 started from that key: ``mix64(key + (i + 1) * GOLDEN)``.
* "Normal" values: the four 16-bit fields of one 64-bit output are summed
  (Irwin-Hall with n = 4), centred and scaled to unit variance.  The integer
  sum is exact and the scaling is ONE float32 multiply by a float32 constant,
  so host and device agree bit for bit.  The distribution has mean 0, variance
  1 and support [-3.46, 3.46]; it stands in for N(0, sigma^2).
* Uniform integers in [0, n): ``((z >> 32) * n) >> 32`` (multiply-shift).
* bf16 values: round-to-nearest-even of the float32 value.
"""
from __future__ import annotations

import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK16 = np.uint64(0xFFFF)

# Irwin-Hall(4) of 16-bit uniforms: mean 4 * 65535 / 2, variance 4 * (65536^2 - 1) / 12.
IH_MEAN = 131070
IH_STD = float(np.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0))

# Tensor ids (stable, documented; the device side receives the derived key).
TID_EMBED = 1
TID_HEAD = 2
TID_TOKENS = 3
TID_EMBEDS_IN = 4


def tid_layer(layer: int, what: str) -> int:
    """Tensor id of a per-layer weight tensor."""
    slot = {"qkv": 0, "o": 1, "gate_up": 2, "down": 3,
            "mhc_w0": 4, "mhc_b0": 5, "mhc_w1": 6, "mhc_b1": 7}[what]
    return 100 + 16 * layer + slot


def tid_kv(slot: int, which: str) -> int:
    """Tensor id of a pre-filled KV slot (which in {'k', 'v'})."""
    return 10000 + 2 * slot + (0 if which == "k" else 1)


def tid_linstate(slot: int, which: str) -> int:
    """Tensor id of a pre-filled linear-attention state (which in {'S', 'z'})."""
    return 20000 + 2 * slot + (0 if which == "S" else 1)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tid: int) -> int:
    """Stream key of tensor (seed, tid): mix64((seed << 32) | tid)."""
    if not (0 <= seed < 2 ** 32 and 0 <= tid < 2 ** 32):
        raise ValueError("seed and tensor id must fit in 32 bits")
    v = np.array([(seed << 32) | tid], dtype=np.uint64)
    with np.errstate(over="ignore"):
        return int(_mix64(v)[0])


def splitmix64_outputs(key: int, start: int, count: int) -> np.ndarray:
    """Outputs start+1 .. start+count of SplitMix64 seeded with ``key``."""
    idx = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(np.uint64(key) + idx * GOLDEN)


def normal_scale(std: float) -> np.float32:
    """The one float32 constant that maps the centred integer sum to value."""
    return np.float32(std / IH_STD)


def _normal_chunk(key: int, start: int, count: int, scale: np.float32) -> np.ndarray:
    z = splitmix64_outputs(key, start, count)
    s = (z & _MASK16) + ((z >> np.uint64(16)) & _MASK16) \
        + ((z >> np.uint64(32)) & _MASK16) + (z >> np.uint64(48))
    centred = (s.astype(np.int64) - IH_MEAN).astype(np.float32)  # exact: |.| < 2^18
    return centred * scale  # one correctly rounded float32 multiply


_POOL = None
_POOL_LOCK = threading.Lock()


def _pool() -> ThreadPoolExecutor:
    global _POOL
    with _POOL_LOCK:
        if _POOL is None:
            n = max(1, min(16, len(os.sched_getaffinity(0))))
            _POOL = ThreadPoolExecutor(max_workers=n)
        return _POOL


def normal_f32(seed: int, tid: int, shape, std: float = 1.0, start: int = 0) -> np.ndarray:
    """float32 array of the given shape: elements start .. start+prod(shape)-1."""
    count = int(np.prod(shape))
    key = stream_key(seed, tid)
    scale = normal_scale(std)
    out = np.empty(count, dtype=np.float32)
    chunk = 1 << 22
    if count <= chunk:
        out[:] = _normal_chunk(key, start, count, scale)
    else:
        def work(off):
            n = min(chunk, count - off)
            out[off:off + n] = _normal_chunk(key, start + off, n, scale)
        list(_pool().map(work, range(0, count, chunk)))
    return out.reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_as_f32(seed: int, tid: int, shape, std: float = 1.0, start: int = 0) -> np.ndarray:
    """The bf16 tensor's values, widened to float32 (exact)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(normal_f32(seed, tid, shape, std, start)))


def abs_normal_f32(seed: int, tid: int, shape, std: float = 1.0, start: int = 0) -> np.ndarray:
    return np.abs(normal_f32(seed, tid, shape, std, start))


def uniform_int(seed: int, tid: int, shape, n: int, start: int = 0) -> np.ndarray:
    """int32 array, uniform in [0, n) (n < 2^31)."""
    if not (0 < n < 2 ** 31):
        raise ValueError("n out of range")
    count = int(np.prod(shape))
    z = splitmix64_outputs(stream_key(seed, tid), start, count)
    with np.errstate(over="ignore"):
        v = ((z >> np.uint64(32)) * np.uint64(n)) >> np.uint64(32)
    return v.astype(np.int32).reshape(shape)


# ----------------------------------------------------------------------------
# Model-level recipes (what each workload draws), shared by tests and bench.
# ----------------------------------------------------------------------------

WEIGHT_STD = 0.02  # every matrix N(0, 0.02); RMSNorm gains are 1


def layer_weight_shapes(hidden, ffn, n_heads, n_kv_heads, head_dim):
    qkv_rows = (n_heads + 2 * n_kv_heads) * head_dim
    return {
        "qkv": (qkv_rows, hidden),
        "o": (hidden, n_heads * head_dim),
        "gate_up": (2 * ffn, hidden),
        "down": (hidden, ffn),
        "mhc_w0": (8, 2 * hidden), "mhc_b0": (8,),
        "mhc_w1": (8, 2 * hidden), "mhc_b1": (8,),
    }
