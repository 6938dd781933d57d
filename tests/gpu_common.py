"""Shared helpers of the GPU tests: build the oracle and the library model from
the same numbers and the same seeded weights."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import looped_weight_shared_loop_amd as L   # loads libloop.so; fails loudly if unbuilt
    return L


def lib_config(ocfg):
    import looped_weight_shared_loop_amd as L
    return L.ModelConfig(vocab=ocfg.vocab, hidden=ocfg.hidden, ffn=ocfg.ffn, n_heads=ocfg.n_heads,
                         n_kv_heads=ocfg.n_kv_heads, head_dim=ocfg.head_dim, n_layers=ocfg.n_layers,
                         loop_start=ocfg.loop_start, loop_end=ocfg.loop_end, n_passes=ocfg.n_passes,
                         sinkhorn_iters=ocfg.sinkhorn_iters, attn_period=ocfg.attn_period,
                         rms_eps=ocfg.rms_eps, la_eps=ocfg.la_eps, dtype=ocfg.dtype)


def mini_bf16_config(**kw):
    """Smallest shape the bf16 kernels accept (head_dim 128, 256-multiples)."""
    base = dict(vocab=1024, hidden=512, ffn=1024, n_heads=4, n_kv_heads=2, head_dim=128,
                n_layers=8, loop_start=2, loop_end=6, n_passes=2, dtype="bf16")
    base.update(kw)
    return oracle.Config(**base)


def tokens(B, S, V, seed=1, start=0):
    return synth.uniform_int(seed, synth.TID_TOKENS, (B, S), V, start=start)


def to_dev_tokens(t):
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).cuda()


def build_pair(ocfg, seed=0, lazy=None, cache_layers=2):
    L = need_gpu()
    gcfg = lib_config(ocfg)
    W = L.random_weights(gcfg, seed)
    model = L.LoopModel(gcfg, W)
    Wo = oracle.make_weights(ocfg, seed, lazy=lazy, cache_layers=cache_layers)
    return model, Wo


def rel(got, ref):
    return oracle.max_row_rel_err(np.asarray(got, np.float64), np.asarray(ref, np.float64))
