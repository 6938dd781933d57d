"""Plain float64 definition of the looped decoder (test infrastructure only).

Abbreviations P1..P5 name the pages; see the package docstring.  Every choice
the pages leave open is a named constant or argument here, and each is listed
with its reading in the repository's design notes (assumptions A1..A24).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from functools import lru_cache
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

import synth

# Where a bf16 configuration stores bf16 (A16): the residual h, the two mHC
# streams X after every write-back, the normed sublayer input u, q/k/v
# (including the KV cache), the attention output, the SwiGLU intermediate and
# every sublayer output y.  Nothing else is rounded.
STORAGE_ROUNDING = ("h", "X", "u", "qkv", "attn", "ffn_inter", "y")


# --------------------------------------------------------------------------
# Configuration and the execution schedule
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    vocab: int
    hidden: int
    ffn: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    loop_start: int
    loop_end: int
    n_passes: int = 2
    sinkhorn_iters: int = 20      # P3 "Two other design pieces"; P5 "What does two-stream mHC do?"
    attn_period: int = 4          # P5 "How does the hybrid attention pattern work?"
    rms_eps: float = 1e-6         # A10
    la_eps: float = 1e-6          # A2
    dtype: str = "fp32"           # "fp32" or "bf16" (A15)
    # bf16 configs round to bf16 at the storage points (A16).  False keeps
    # float64 between the steps instead, on the same bf16-valued weights and
    # inputs: the exact-arithmetic result that bf16 storage approximates,
    # which measures how far rounding alone moves an output.
    round_storage: bool = True

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


def tiny_config(**kw) -> Config:
    """The tiny looped decoder: 8 stored layers, block [2, 6) run twice, fp32."""
    base = dict(vocab=512, hidden=256, ffn=768, n_heads=4, n_kv_heads=4, head_dim=64,
                n_layers=8, loop_start=2, loop_end=6, n_passes=2, dtype="fp32")
    base.update(kw)
    return Config(**base)


def nine_b_config(**kw) -> Config:
    """The Loop-9B shape: 32 stored layers, block [4, 28) run twice
    (P1 "The trick"; P3 "Key specs from the card": hidden 4,096, FFN 12,288,
    vocabulary 248,320); heads 32 q / 8 kv of dim 128 (A3)."""
    base = dict(vocab=248320, hidden=4096, ffn=12288, n_heads=32, n_kv_heads=8, head_dim=128,
                n_layers=32, loop_start=4, loop_end=28, n_passes=2, dtype="bf16")
    base.update(kw)
    return Config(**base)


def group_config(**kw) -> Config:
    """One 4-layer group [linear, linear, linear, full] at 9B width, looped twice."""
    base = dict(vocab=248320, hidden=4096, ffn=12288, n_heads=32, n_kv_heads=8, head_dim=128,
                n_layers=4, loop_start=0, loop_end=4, n_passes=2, dtype="bf16")
    base.update(kw)
    return Config(**base)


def layer_is_full(cfg: Config, layer: int) -> bool:
    """Three linear-attention layers then one full-attention layer per group of
    ``attn_period`` stored layers (P3 "Two other design pieces"; P5 "How does the
    hybrid attention pattern work?").  Decided by the stored index (A1)."""
    return layer % cfg.attn_period == cfg.attn_period - 1


def in_loop(cfg: Config, layer: int) -> bool:
    return cfg.loop_start <= layer < cfg.loop_end


def schedule(cfg: Config) -> List[Tuple[int, int]]:
    """Execution order as (stored layer, pass): layers before the block once,
    the block ``n_passes`` times with each pass fed the previous pass's output,
    then the rest once (P1 "The trick"; P5 "What is the looped decoder ...?",
    steps 1-4).  Pass index is 0 outside the block."""
    s = [(i, 0) for i in range(cfg.loop_start)]
    for p in range(cfg.n_passes):
        s += [(i, p) for i in range(cfg.loop_start, cfg.loop_end)]
    s += [(i, 0) for i in range(cfg.loop_end, cfg.n_layers)]
    return s


# --------------------------------------------------------------------------
# Weights (random init; lazily generated for the wide shapes)
# --------------------------------------------------------------------------

@dataclass
class LayerWeights:
    attn_norm: np.ndarray          # [C] fp32 gain
    ffn_norm: np.ndarray           # [C] fp32 gain
    qkv: np.ndarray                # [(Hq + 2 Hkv) d, C]: q rows, then k rows, then v rows
    o: np.ndarray                  # [C, Hq d]
    gate_up: np.ndarray            # [2F, C]: gate rows, then up rows
    down: np.ndarray               # [C, F]
    mhc_w: Optional[List[np.ndarray]] = None   # per site (attention, FFN): [8, 2C] fp32
    mhc_b: Optional[List[np.ndarray]] = None   # per site: [8] fp32


class Weights:
    """Weights of one model.  ``layers`` may be a list or a callable
    ``layer -> LayerWeights`` (lazy).  Embedding rows and head rows can come
    from callables too, so the 9B shape never needs all 8B values at once."""

    def __init__(self, cfg: Config, layers, embed=None, head=None, final_norm=None,
                 embed_rows: Optional[Callable] = None, head_rows: Optional[Callable] = None):
        self.cfg = cfg
        self._layers = layers
        self.embed = embed
        self.head = head
        self.final_norm = final_norm if final_norm is not None else np.ones(cfg.hidden, np.float32)
        self._embed_rows = embed_rows
        self._head_rows = head_rows

    def layer(self, i: int) -> LayerWeights:
        if callable(self._layers):
            return self._layers(i)
        return self._layers[i]

    def embed_rows(self, tokens: np.ndarray) -> np.ndarray:
        if self.embed is not None:
            return self.embed[tokens]
        return self._embed_rows(tokens)

    def head_blocks(self, block: int = 16384):
        """Yields (row0, W_head[row0:row1]) blocks."""
        V = self.cfg.vocab
        if self.head is not None:
            yield 0, self.head
            return
        for r0 in range(0, V, block):
            yield r0, self._head_rows(r0, min(V, r0 + block))


def _gen(cfg: Config, seed: int, tid: int, shape, start: int = 0) -> np.ndarray:
    if cfg.dtype == "bf16":
        return synth.normal_bf16_as_f32(seed, tid, shape, synth.WEIGHT_STD, start)
    return synth.normal_f32(seed, tid, shape, synth.WEIGHT_STD, start)


def make_layer(cfg: Config, seed: int, i: int) -> LayerWeights:
    shp = synth.layer_weight_shapes(cfg.hidden, cfg.ffn, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim)
    L = LayerWeights(
        attn_norm=np.ones(cfg.hidden, np.float32), ffn_norm=np.ones(cfg.hidden, np.float32),
        qkv=_gen(cfg, seed, synth.tid_layer(i, "qkv"), shp["qkv"]),
        o=_gen(cfg, seed, synth.tid_layer(i, "o"), shp["o"]),
        gate_up=_gen(cfg, seed, synth.tid_layer(i, "gate_up"), shp["gate_up"]),
        down=_gen(cfg, seed, synth.tid_layer(i, "down"), shp["down"]))
    if in_loop(cfg, i):
        # mHC parameters are float32 whatever the backbone dtype (P5 "What are the key specs?").
        L.mhc_w = [synth.normal_f32(seed, synth.tid_layer(i, f"mhc_w{s}"), shp[f"mhc_w{s}"], synth.WEIGHT_STD)
                   for s in (0, 1)]
        L.mhc_b = [synth.normal_f32(seed, synth.tid_layer(i, f"mhc_b{s}"), shp[f"mhc_b{s}"], synth.WEIGHT_STD)
                   for s in (0, 1)]
    return L


def make_weights(cfg: Config, seed: int = 0, lazy: Optional[bool] = None, cache_layers: int = 2) -> Weights:
    """Random-init weights: every matrix (and mHC bias) ~ N(0, 0.02) from
    ``synth``; RMSNorm gains 1 (A17)."""
    if lazy is None:
        lazy = cfg.vocab * cfg.hidden > (1 << 26)
    if not lazy:
        embed = _gen(cfg, seed, synth.TID_EMBED, (cfg.vocab, cfg.hidden))
        head = _gen(cfg, seed, synth.TID_HEAD, (cfg.vocab, cfg.hidden))
        layers = [make_layer(cfg, seed, i) for i in range(cfg.n_layers)]
        return Weights(cfg, layers, embed=embed, head=head)

    layer_fn = lru_cache(maxsize=cache_layers)(lambda i: make_layer(cfg, seed, i))
    C = cfg.hidden

    def embed_rows(tokens):
        flat = np.asarray(tokens).reshape(-1)
        out = np.empty((flat.size, C), np.float32)
        for j, t in enumerate(flat):
            out[j] = _gen(cfg, seed, synth.TID_EMBED, (C,), start=int(t) * C)
        return out.reshape(np.asarray(tokens).shape + (C,))

    def head_rows(r0, r1):
        return _gen(cfg, seed, synth.TID_HEAD, (r1 - r0, C), start=r0 * C)

    return Weights(cfg, layer_fn, embed_rows=embed_rows, head_rows=head_rows)


# --------------------------------------------------------------------------
# Primitive steps
# --------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even), returned as float64.  Written with
    integer operations on the float32 bit pattern."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _store(cfg: Config, x: np.ndarray) -> np.ndarray:
    """Value as the GPU path stores it: bf16 for bf16 configs (unless
    ``round_storage`` is off), exact otherwise."""
    if cfg.dtype == "bf16" and cfg.round_storage:
        return round_bf16(x)
    return np.asarray(x, dtype=np.float64)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """gamma * x / sqrt(mean(x^2) + eps) over the last axis (A10)."""
    x = np.asarray(x, dtype=np.float64)
    return np.asarray(gamma, np.float64) * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def elu_plus_one(x):
    """Feature map of the linear attention (A2): elu(x) + 1."""
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def sinkhorn(M: np.ndarray, iters: int) -> np.ndarray:
    """Sinkhorn normalisation of positive matrices ``M[..., n, n]``: each
    iteration divides every row by its sum, then every column by its sum
    (P5 "What does two-stream mHC do?"; order per A7)."""
    M = np.asarray(M, dtype=np.float64)
    for _ in range(iters):
        M = M / M.sum(axis=-1, keepdims=True)
        M = M / M.sum(axis=-2, keepdims=True)
    return M


def mhc_maps(X: np.ndarray, w: np.ndarray, b: np.ndarray, iters: int, eps: float):
    """Per-token maps of one mHC site from the two streams ``X[..., 2, C]``
    (P3 "Two other design pieces"; P5 "What does two-stream mHC do?"; A6, A7).

    x_hat = vec(X) / rms(vec(X)) with vec = [stream 0, stream 1];
    l = W x_hat + b (8 values, order pre0 pre1 post0 post1 r00 r01 r10 r11);
    H_pre = sigmoid(l0, l1), H_post = 2 sigmoid(l2, l3),
    H_res = Sinkhorn_iters(exp(R - max R)), R = [[l4, l5], [l6, l7]].
    Returns (H_pre [..., 2], H_post [..., 2], H_res [..., 2, 2], logits [..., 8]).
    """
    X = np.asarray(X, dtype=np.float64)
    flat = X.reshape(X.shape[:-2] + (-1,))
    xhat = flat / np.sqrt(np.mean(flat * flat, axis=-1, keepdims=True) + eps)
    logits = xhat @ np.asarray(w, np.float64).T + np.asarray(b, np.float64)
    pre = sigmoid(logits[..., 0:2])
    post = 2.0 * sigmoid(logits[..., 2:4])
    R = logits[..., 4:8].reshape(logits.shape[:-1] + (2, 2))
    M = np.exp(R - R.max(axis=(-1, -2), keepdims=True))
    return pre, post, sinkhorn(M, iters), logits


def full_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, pos0: int) -> np.ndarray:
    """Causal softmax attention with grouped KV heads (P5 "How does the hybrid
    attention pattern work?"; A3, A12, A23).

    q [B, T, Hq, d] are positions pos0 .. pos0+T-1; k, v [B, S, Hkv, d] are
    positions 0 .. S-1.  Query head j reads KV head j // (Hq / Hkv); scores are
    q.k / sqrt(d); key tau is visible to query t iff tau <= pos0 + t.
    """
    B, T, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    out = np.empty((B, T, Hq, d), np.float64)
    qpos = pos0 + np.arange(T)[:, None]
    visible = np.arange(S)[None, :] <= qpos
    for bb in range(B):
        for j in range(Hq):
            kv = j // g
            s = (q[bb, :, j, :].astype(np.float64) @ k[bb, :, kv, :].astype(np.float64).T) / math.sqrt(d)
            s = np.where(visible, s, -np.inf)
            p = np.exp(s - s.max(axis=-1, keepdims=True))
            p = p / p.sum(axis=-1, keepdims=True)
            out[bb, :, j, :] = p @ v[bb, :, kv, :].astype(np.float64)
    return out


def linear_attention(q, k, v, S0, z0, eps: float):
    """Causal linear attention with the elu+1 feature map and a normaliser,
    carried as a fixed-size state (P5 "How does the hybrid attention pattern
    work?"; variant per A2), written as its recurrence:

        S_t = S_{t-1} + phi(k_t) v_t^T,  z_t = z_{t-1} + phi(k_t),
        o_t = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps),

    per KV head; query head j reads the state of KV head j // (Hq / Hkv).
    q [B, T, Hq, d]; k, v [B, T, Hkv, d]; S0 [B, Hkv, d, d]; z0 [B, Hkv, d].
    Returns (o [B, T, Hq, d], S_T, z_T).
    """
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    S = np.array(S0, dtype=np.float64)
    z = np.array(z0, dtype=np.float64)
    out = np.empty((B, T, Hq, d), np.float64)
    for t in range(T):
        fk = elu_plus_one(np.asarray(k[:, t], np.float64))              # [B, Hkv, d]
        S = S + fk[..., :, None] * np.asarray(v[:, t], np.float64)[..., None, :]
        z = z + fk
        fq = elu_plus_one(np.asarray(q[:, t], np.float64)).reshape(B, Hkv, g, d)
        num = np.einsum("bhgi,bhij->bhgj", fq, S)
        den = np.einsum("bhgi,bhi->bhg", fq, z) + eps
        out[:, t] = (num / den[..., None]).reshape(B, Hq, d)
    return out, S, z


def swiglu_ffn(cfg: Config, u: np.ndarray, gate_up: np.ndarray, down: np.ndarray) -> np.ndarray:
    """y = W_down (silu(W_gate u) * (W_up u)) (P3 "Key specs": FFN 12,288; A10)."""
    F = cfg.ffn
    gu = u @ np.asarray(gate_up, np.float64).T
    inter = _store(cfg, silu(gu[..., :F]) * gu[..., F:])
    return _store(cfg, inter @ np.asarray(down, np.float64).T)


# --------------------------------------------------------------------------
# Per-(layer, pass) state: KV caches and linear-attention states (A13, A14)
# --------------------------------------------------------------------------

@dataclass
class State:
    length: int = 0
    kv: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]] = field(default_factory=dict)
    lin: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]] = field(default_factory=dict)
    calls: List[Tuple[int, int, str]] = field(default_factory=list)   # (layer, pass, sublayer)


def attention_sublayer(cfg: Config, u, L: LayerWeights, layer: int, pss: int, st: State, pos0: int):
    B, T, _ = u.shape
    Hq, Hkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    qkv = _store(cfg, u @ np.asarray(L.qkv, np.float64).T)
    q = qkv[..., :Hq * d].reshape(B, T, Hq, d)
    k = qkv[..., Hq * d:(Hq + Hkv) * d].reshape(B, T, Hkv, d)
    v = qkv[..., (Hq + Hkv) * d:].reshape(B, T, Hkv, d)
    key = (layer, pss)
    if layer_is_full(cfg, layer):
        if key in st.kv:
            k = np.concatenate([st.kv[key][0], k], axis=1)
            v = np.concatenate([st.kv[key][1], v], axis=1)
        st.kv[key] = (k, v)
        a = full_attention(q, k, v, pos0)
        st.calls.append((layer, pss, "full"))
    else:
        S0, z0 = st.lin.get(key, (np.zeros((B, Hkv, d, d)), np.zeros((B, Hkv, d))))
        a, S1, z1 = linear_attention(q, k, v, S0, z0, cfg.la_eps)
        st.lin[key] = (S1, z1)
        st.calls.append((layer, pss, "linear"))
    a = _store(cfg, a.reshape(B, T, Hq * d))
    return _store(cfg, a @ np.asarray(L.o, np.float64).T)


def ffn_sublayer(cfg: Config, u, L: LayerWeights, layer: int, pss: int, st: State):
    st.calls.append((layer, pss, "ffn"))
    return swiglu_ffn(cfg, u, L.gate_up, L.down)


def plain_layer(cfg, h, L, layer, pss, st, pos0):
    """A layer outside the looped block: two pre-norm residual sublayers
    h <- h + f(RMSNorm(h)) (A9, A10)."""
    u = _store(cfg, rmsnorm(h, L.attn_norm, cfg.rms_eps))
    h = _store(cfg, h + attention_sublayer(cfg, u, L, layer, pss, st, pos0))
    u = _store(cfg, rmsnorm(h, L.ffn_norm, cfg.rms_eps))
    return _store(cfg, h + ffn_sublayer(cfg, u, L, layer, pss, st))


def mhc_site(cfg, X, w, b, gamma, f):
    """One two-stream hyper-connection site (P5 "What does two-stream mHC do?":
    how the layer reads the streams, how they mix, how its output is written
    back; placed per sublayer, A5):

        x_in = H_pre0 X0 + H_pre1 X1,   y = f(RMSNorm(x_in)),
        X_i <- sum_j H_res[i, j] X_j + H_post[i] y.
    """
    pre, post, res, _ = mhc_maps(X, w, b, cfg.sinkhorn_iters, cfg.rms_eps)
    x_in = pre[..., 0:1] * X[..., 0, :] + pre[..., 1:2] * X[..., 1, :]
    u = _store(cfg, rmsnorm(x_in, gamma, cfg.rms_eps))
    y = f(u)
    mixed = np.einsum("...ij,...jc->...ic", res, X)
    return _store(cfg, mixed + post[..., :, None] * y[..., None, :])


def looped_layer(cfg, X, L, layer, pss, st, pos0):
    X = mhc_site(cfg, X, L.mhc_w[0], L.mhc_b[0], L.attn_norm,
                 lambda u: attention_sublayer(cfg, u, L, layer, pss, st, pos0))
    X = mhc_site(cfg, X, L.mhc_w[1], L.mhc_b[1], L.ffn_norm,
                 lambda u: ffn_sublayer(cfg, u, L, layer, pss, st))
    return X


# --------------------------------------------------------------------------
# The forward pass
# --------------------------------------------------------------------------

def forward(cfg: Config, W: Weights, tokens: Optional[np.ndarray] = None,
            embeds: Optional[np.ndarray] = None, state: Optional[State] = None,
            all_logits: bool = False, hidden_out: bool = False):
    """Forward over T new positions of B sequences, continuing ``state``.

    tokens [B, T] int (or embeds [B, T, C] given directly).  Returns logits
    [B, V] for the last position, [B, T, V] with ``all_logits``, or the final
    residual h [B, T, C] with ``hidden_out`` (before the final norm).  Streams
    enter the looped block as two copies of h and leave it as their mean, once
    per forward, not once per pass (A4).
    """
    st = state if state is not None else State()
    pos0 = st.length
    if embeds is not None:
        h = _store(cfg, np.asarray(embeds, np.float64))
    else:
        h = np.asarray(W.embed_rows(np.asarray(tokens)), np.float64)
    X = None
    for layer, pss in schedule(cfg):
        L = W.layer(layer)
        if in_loop(cfg, layer):
            if layer == cfg.loop_start and pss == 0:
                X = np.stack([h, h], axis=-2)                       # enter: copy h to both streams
            X = looped_layer(cfg, X, L, layer, pss, st, pos0)
            if layer == cfg.loop_end - 1 and pss == cfg.n_passes - 1:
                h = _store(cfg, 0.5 * (X[..., 0, :] + X[..., 1, :]))  # exit: mean of the streams
        else:
            h = plain_layer(cfg, h, L, layer, pss, st, pos0)
    st.length = pos0 + h.shape[1]
    if hidden_out:
        return h
    rows = h if all_logits else h[:, -1:, :]
    u = _store(cfg, rmsnorm(rows, W.final_norm, cfg.rms_eps))
    logits = np.empty(u.shape[:-1] + (cfg.vocab,), np.float64)
    for r0, blk in W.head_blocks():
        logits[..., r0:r0 + blk.shape[0]] = u @ np.asarray(blk, np.float64).T
    return logits if all_logits else logits[:, 0, :]


def max_row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over output rows of ||got - ref||_inf / ||ref||_inf (A18)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    g2 = got.reshape(-1, got.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    num = np.abs(g2 - r2).max(axis=-1)
    den = np.abs(r2).max(axis=-1)
    return float((num / np.maximum(den, 1e-300)).max())
