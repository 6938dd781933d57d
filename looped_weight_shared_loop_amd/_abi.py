"""ctypes binding of libloop.so (include/loop.h), one Python function per C
entry point, same names.  Argument marshalling only: every step of the forward
pass runs in the library's HIP kernels.  Raises ``LoopError`` on a non-zero
status.  Loading fails loudly when the library has not been built."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_size_t, c_uint, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libloop.so")

LOOP_OK = 0
LOOP_ERR_INVALID_ARG = -1
LOOP_ERR_SHAPE = -2
LOOP_ERR_ALIGN = -3
LOOP_ERR_CAPACITY = -4
LOOP_ERR_WORKSPACE = -5
LOOP_ERR_NO_DEVICE = -6
LOOP_ERR_HIP = -7
LOOP_ERR_DEVICE_FLAG = -8
LOOP_ERR_STATE = -9

LOOP_FP32 = 0
LOOP_BF16 = 1

LOOP_ALL_LOGITS = 1
LOOP_HIDDEN_OUT = 2
LOOP_CONTINUE = 4

REGION_K, REGION_VT, REGION_S, REGION_Z, REGION_HEADER = 0, 1, 2, 3, 4


class LoopError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {msg} (status {code})")
        self.code = code


class loop_config(ctypes.Structure):
    _fields_ = [("vocab", c_int), ("hidden", c_int), ("ffn", c_int), ("n_heads", c_int),
                ("n_kv_heads", c_int), ("head_dim", c_int), ("n_layers", c_int),
                ("loop_start", c_int), ("loop_end", c_int), ("n_passes", c_int),
                ("sinkhorn_iters", c_int), ("attn_period", c_int), ("rms_eps", c_float),
                ("la_eps", c_float), ("dtype", c_int)]


class loop_layer_weights(ctypes.Structure):
    _fields_ = [("attn_norm", c_void_p), ("ffn_norm", c_void_p), ("qkv", c_void_p), ("o", c_void_p),
                ("gate_up", c_void_p), ("down", c_void_p), ("mhc_w", c_void_p * 2), ("mhc_b", c_void_p * 2)]


class loop_weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("final_norm", c_void_p), ("head", c_void_p),
                ("layers", POINTER(loop_layer_weights)), ("n_layers", c_int)]


SYMBOLS = {
    # name: (restype, argtypes)
    "loop_model_create": (c_int, [POINTER(loop_config), POINTER(loop_weights), POINTER(c_void_p)]),
    "loop_model_destroy": (c_int, [c_void_p]),
    "loop_model_schedule": (c_int, [c_void_p, c_int, POINTER(c_int), POINTER(c_int), POINTER(c_int),
                                    POINTER(c_int), POINTER(c_int)]),
    "loop_state_bytes": (c_int, [c_void_p, c_int, c_int, POINTER(c_size_t)]),
    "loop_workspace_bytes": (c_int, [c_void_p, c_int, c_int, c_int, POINTER(c_size_t)]),
    "loop_state_create": (c_int, [c_void_p, c_void_p, c_size_t, c_int, c_int, POINTER(c_void_p)]),
    "loop_state_bytes_paged": (c_int, [c_void_p, c_int, c_int, c_int, POINTER(c_size_t)]),
    "loop_state_create_paged": (c_int, [c_void_p, c_void_p, c_size_t, c_int, c_int, c_int, c_void_p,
                                        POINTER(c_void_p)]),
    "loop_state_destroy": (c_int, [c_void_p]),
    "loop_state_length": (c_int, [c_void_p, POINTER(c_int)]),
    "loop_state_set_length": (c_int, [c_void_p, c_int]),
    "loop_state_seq_length": (c_int, [c_void_p, c_int, POINTER(c_int)]),
    "loop_state_set_seq_length": (c_int, [c_void_p, c_int, c_int]),
    "loop_state_region": (c_int, [c_void_p, c_int, c_int, POINTER(c_void_p), POINTER(c_size_t)]),
    "loop_state_check": (c_int, [c_void_p, c_void_p]),
    "loop_prefill": (c_int, [c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p, c_int, c_int,
                             c_uint, c_void_p, c_void_p]),
    "loop_prefill_rows": (c_int, [c_void_p, c_void_p, c_void_p, c_size_t, c_int, c_void_p, c_void_p, c_int, c_int,
                                  c_uint, c_void_p, c_void_p]),
    "loop_decode_step": (c_int, [c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_int, c_void_p, c_void_p]),
    "loop_decode_pipelined": (c_int, [c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_int, c_void_p, c_void_p,
                                      c_void_p]),
    "loop_decode_step_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p]),
    "loop_status_string": (ctypes.c_char_p, [c_int]),
    "loop_last_error": (ctypes.c_char_p, []),
    # op level (include/loop_ops.h)
    "loop_op_gemm_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "loop_op_gemm": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, ctypes.c_long, c_void_p, ctypes.c_long,
                             c_void_p, ctypes.c_long, c_int, c_void_p, c_size_t, c_void_p]),
    "loop_op_add_rmsnorm": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_void_p]),
    "loop_op_mhc_bytes": (c_size_t, [c_int]),
    "loop_op_mhc": (c_int, [c_int, c_int, c_int, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "loop_op_attention": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, ctypes.c_long,
                                  c_void_p, c_void_p, c_void_p, ctypes.c_long, c_void_p]),
    "loop_op_attention_decode_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "loop_op_attention_decode": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p,
                                         ctypes.c_long, c_void_p, c_void_p, c_void_p, ctypes.c_long, c_void_p,
                                         c_size_t, c_void_p]),
    "loop_op_attention_decode_ragged": (c_int, [c_int, c_int, c_int, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                                c_void_p, ctypes.c_long, c_void_p, c_void_p, c_void_p, ctypes.c_long,
                                                c_void_p, c_size_t, c_void_p]),
    "loop_op_attention_decode_stream_k_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "loop_op_attention_decode_stream_k": (c_int, [c_int, c_int, c_int, c_void_p, c_int, c_int, c_int, c_int,
                                                  c_void_p, ctypes.c_long, c_void_p, c_void_p, c_void_p,
                                                  ctypes.c_long, c_void_p, c_size_t, c_void_p]),
    "loop_op_linear_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
    "loop_op_linear": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_void_p, ctypes.c_long,
                               c_void_p, c_void_p, c_int, c_void_p, ctypes.c_long, c_void_p, c_size_t, c_void_p]),
}

LOOP_EPI_STORE, LOOP_EPI_F32, LOOP_EPI_SWIGLU = 0, 1, 3
LOOP_MHC_ENTER, LOOP_MHC_MID, LOOP_MHC_EXIT = 0, 1, 2

_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python looped_weight_shared_loop_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SYMBOLS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(code: int, where: str):
    if code != LOOP_OK:
        msg = lib().loop_last_error().decode(errors="replace")
        raise LoopError(code, where, msg)


def loop_status_string(code: int) -> str:
    return lib().loop_status_string(code).decode()


def loop_last_error() -> str:
    return lib().loop_last_error().decode(errors="replace")


def loop_model_create(cfg: loop_config, weights: loop_weights) -> c_void_p:
    h = c_void_p()
    _check(lib().loop_model_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(h)), "loop_model_create")
    return h


def loop_model_destroy(m) -> None:
    _check(lib().loop_model_destroy(m), "loop_model_destroy")


def loop_model_schedule(m):
    n = c_int()
    _check(lib().loop_model_schedule(m, 0, None, None, None, None, ctypes.byref(n)), "loop_model_schedule")
    arrs = [(c_int * n.value)() for _ in range(4)]
    _check(lib().loop_model_schedule(m, n.value, *arrs, ctypes.byref(n)), "loop_model_schedule")
    return [tuple(a[e] for a in arrs) for e in range(n.value)]   # (layer, pass, kind, slot)


def loop_state_bytes(m, batch: int, max_seq: int) -> int:
    b = c_size_t()
    _check(lib().loop_state_bytes(m, batch, max_seq, ctypes.byref(b)), "loop_state_bytes")
    return b.value


def loop_workspace_bytes(m, batch: int, max_tokens: int, max_seq: int) -> int:
    b = c_size_t()
    _check(lib().loop_workspace_bytes(m, batch, max_tokens, max_seq, ctypes.byref(b)), "loop_workspace_bytes")
    return b.value


def loop_state_create(m, state_ptr: int, nbytes: int, batch: int, max_seq: int) -> c_void_p:
    h = c_void_p()
    _check(lib().loop_state_create(m, c_void_p(state_ptr), nbytes, batch, max_seq, ctypes.byref(h)),
           "loop_state_create")
    return h


def loop_state_bytes_paged(m, batch: int, max_seq: int, n_pages: int) -> int:
    b = c_size_t()
    _check(lib().loop_state_bytes_paged(m, batch, max_seq, n_pages, ctypes.byref(b)), "loop_state_bytes_paged")
    return b.value


def loop_state_create_paged(m, state_ptr: int, nbytes: int, batch: int, max_seq: int, n_pages: int,
                            table_ptr: int) -> c_void_p:
    h = c_void_p()
    _check(lib().loop_state_create_paged(m, c_void_p(state_ptr), nbytes, batch, max_seq, n_pages,
                                         c_void_p(table_ptr), ctypes.byref(h)), "loop_state_create_paged")
    return h


def loop_state_destroy(st) -> None:
    _check(lib().loop_state_destroy(st), "loop_state_destroy")


def loop_state_length(st) -> int:
    n = c_int()
    _check(lib().loop_state_length(st, ctypes.byref(n)), "loop_state_length")
    return n.value


def loop_state_set_length(st, length: int) -> None:
    _check(lib().loop_state_set_length(st, length), "loop_state_set_length")


def loop_state_seq_length(st, seq: int) -> int:
    n = c_int()
    _check(lib().loop_state_seq_length(st, seq, ctypes.byref(n)), "loop_state_seq_length")
    return n.value


def loop_state_set_seq_length(st, seq: int, length: int) -> None:
    _check(lib().loop_state_set_seq_length(st, seq, length), "loop_state_set_seq_length")


def loop_state_region(st, kind: int, slot: int):
    p = c_void_p()
    n = c_size_t()
    _check(lib().loop_state_region(st, kind, slot, ctypes.byref(p), ctypes.byref(n)), "loop_state_region")
    return p.value, n.value


def loop_state_check(st, stream: int) -> None:
    _check(lib().loop_state_check(st, c_void_p(stream)), "loop_state_check")


def loop_prefill(m, st, ws_ptr: int, ws_bytes: int, tokens_ptr, embeds_ptr, B: int, S: int, flags: int,
                 out_ptr: int, stream: int) -> None:
    _check(lib().loop_prefill(m, st, c_void_p(ws_ptr), ws_bytes, c_void_p(tokens_ptr), c_void_p(embeds_ptr),
                              B, S, flags, c_void_p(out_ptr), c_void_p(stream)), "loop_prefill")


def loop_prefill_rows(m, st, ws_ptr: int, ws_bytes: int, seq0: int, tokens_ptr, embeds_ptr, B: int, S: int,
                      flags: int, out_ptr: int, stream: int) -> None:
    _check(lib().loop_prefill_rows(m, st, c_void_p(ws_ptr), ws_bytes, seq0, c_void_p(tokens_ptr),
                                   c_void_p(embeds_ptr), B, S, flags, c_void_p(out_ptr), c_void_p(stream)),
           "loop_prefill_rows")


def loop_decode_step(m, st, ws_ptr: int, ws_bytes: int, tokens_ptr: int, B: int, logits_ptr: int,
                     stream: int) -> None:
    _check(lib().loop_decode_step(m, st, c_void_p(ws_ptr), ws_bytes, c_void_p(tokens_ptr), B,
                                  c_void_p(logits_ptr), c_void_p(stream)), "loop_decode_step")


def loop_decode_step_noalloc(m, st, tokens_ptr: int, B: int, logits_ptr: int, stream: int) -> None:
    _check(lib().loop_decode_step_noalloc(m, st, c_void_p(tokens_ptr), B, c_void_p(logits_ptr), c_void_p(stream)),
           "loop_decode_step_noalloc")


LOOP_NOALLOC_WORKSPACE_BYTES = 64 << 20


def loop_decode_pipelined(m, st, ws_ptr: int, ws_bytes: int, tokens_ptr, B: int, logits_ptr, stream: int):
    """Returns (entered cohort, cohort whose logits were written), -1 for none."""
    info = (c_int * 2)(-1, -1)
    _check(lib().loop_decode_pipelined(m, st, c_void_p(ws_ptr), ws_bytes, c_void_p(tokens_ptr), B,
                                       c_void_p(logits_ptr), info, c_void_p(stream)), "loop_decode_pipelined")
    return int(info[0]), int(info[1])


# ---------------------------------------------------------------- op level

def _p(x):
    return None if x is None else c_void_p(x)


def loop_op_gemm_bytes(dtype, epi, M, N, K, F) -> int:
    return lib().loop_op_gemm_bytes(dtype, epi, M, N, K, F)


def loop_op_gemm(dtype, epi, M, N, K, A, lda, B, ldb, C, ldc, F, stream, scratch=None, scratch_bytes=0) -> None:
    _check(lib().loop_op_gemm(dtype, epi, M, N, K, _p(A), lda, _p(B), ldb, _p(C), ldc, F, _p(scratch), scratch_bytes,
                              _p(stream)), "loop_op_gemm")


def loop_op_add_rmsnorm(dtype, T, C, y, h, gamma, u, eps, stream) -> None:
    _check(lib().loop_op_add_rmsnorm(dtype, T, C, _p(y), _p(h), _p(gamma), _p(u), eps, _p(stream)),
           "loop_op_add_rmsnorm")


def loop_op_mhc_bytes(C) -> int:
    return lib().loop_op_mhc_bytes(C)


def loop_op_mhc(dtype, mode, T, C, iters, eps, y, h, X, maps_in, maps_out, w, b, gamma, u, scratch, nbytes,
                stream) -> None:
    _check(lib().loop_op_mhc(dtype, mode, T, C, iters, eps, _p(y), _p(h), _p(X), _p(maps_in), _p(maps_out), _p(w),
                             _p(b), _p(gamma), _p(u), _p(scratch), nbytes, _p(stream)), "loop_op_mhc")


def loop_op_attention(dtype, B, S, pos0, S_max, Hq, Hkv, d, q, ldq, k, v, out, ldo, stream) -> None:
    _check(lib().loop_op_attention(dtype, B, S, pos0, S_max, Hq, Hkv, d, _p(q), ldq, _p(k), _p(v), _p(out), ldo,
                                   _p(stream)), "loop_op_attention")


def loop_op_attention_decode_bytes(B, S, Hq, d, S_max) -> int:
    return lib().loop_op_attention_decode_bytes(B, S, Hq, d, S_max)


def loop_op_attention_decode(dtype, B, S, pos0, S_max, Hq, Hkv, d, q, ldq, k, v, out, ldo, scratch, nbytes,
                             stream) -> None:
    _check(lib().loop_op_attention_decode(dtype, B, S, pos0, S_max, Hq, Hkv, d, _p(q), ldq, _p(k), _p(v), _p(out),
                                          ldo, _p(scratch), nbytes, _p(stream)), "loop_op_attention_decode")


def loop_op_attention_decode_ragged(dtype, B, S, pos, max_pos0, S_max, Hq, Hkv, d, q, ldq, k, v, out, ldo, scratch,
                                    nbytes, stream) -> None:
    _check(lib().loop_op_attention_decode_ragged(dtype, B, S, _p(pos), max_pos0, S_max, Hq, Hkv, d, _p(q), ldq, _p(k),
                                                 _p(v), _p(out), ldo, _p(scratch), nbytes, _p(stream)),
           "loop_op_attention_decode_ragged")


def loop_op_attention_decode_stream_k_bytes(B, S, Hq, Hkv, d) -> int:
    return lib().loop_op_attention_decode_stream_k_bytes(B, S, Hq, Hkv, d)


def loop_op_attention_decode_stream_k(dtype, B, S, starts, S_max, Hq, Hkv, d, q, ldq, k, v, out, ldo, scratch, nbytes,
                                      stream) -> None:
    """starts: host address of an int32 array of the B first new positions (e.g. numpy `a.ctypes.data`)."""
    _check(lib().loop_op_attention_decode_stream_k(dtype, B, S, _p(starts), S_max, Hq, Hkv, d, _p(q), ldq, _p(k),
                                                   _p(v), _p(out), ldo, _p(scratch), nbytes, _p(stream)),
           "loop_op_attention_decode_stream_k")


def loop_op_linear_bytes(B, S, Hkv, d) -> int:
    return lib().loop_op_linear_bytes(B, S, Hkv, d)


def loop_op_linear(dtype, chunked, B, S, Hq, Hkv, d, eps, qkv, ld, S_state, z_state, init_zero, out, ldo, scratch,
                   nbytes, stream) -> None:
    _check(lib().loop_op_linear(dtype, chunked, B, S, Hq, Hkv, d, eps, _p(qkv), ld, _p(S_state), _p(z_state),
                                init_zero, _p(out), ldo, _p(scratch), nbytes, _p(stream)), "loop_op_linear")
