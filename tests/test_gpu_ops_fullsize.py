"""Full-size parity of each kernel family, in the launch configuration the
9B-shape prefill and decode use, on sampled outputs the oracle recomputes one
by one (inputs drawn on the device by the seeded generator and redrawn on the
host for the sampled rows only).

Bars (element-wise unless stated):
  GEMM, float32 out   |g - r| <= 1e-5 * sum_k |a_k b_k|        (fp32 accumulation)
  GEMM, bf16 out      |g - r| <= 2^-8 |r| + 1e-5 * sum_k |a_k b_k|  (one bf16 rounding)
  mHC                 X' within 1 bf16 ulp (<= 2^-7 |x|), u within 2 ulp; maps of the kernel's own X'
                      within 2e-6 (float32-equivalent projection)
  attention (bf16)    per query row ||g - r||_inf <= 2e-2 ||r||_inf (probabilities rounded to bf16)
  linear attention    per row ||g - r||_inf <= 1e-2 ||r||_inf; state rel 1e-4
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import model as M
from gpu_common import need_gpu, torch

pytestmark = pytest.mark.gpu

C, F, V = 4096, 12288, 248320
HQ, HKV, D = 32, 8, 128
QKV = (HQ + 2 * HKV) * D
SEED = 7
# attention head layouts at 9B width: 32 query / 8 KV heads of 128, and the
# 16 / 4 heads of 256 of "How Does SenseNova-Loop Get More Depth Without More
# Parameters?" (section on the hybrid attention pattern); same projection sizes
LAYOUTS = {"32x128": (32, 8, 128), "16x256": (16, 4, 256)}


def _lay(layout):
    hq, hkv, d = LAYOUTS[layout]
    return hq, hkv, d, (hq + 2 * hkv) * d


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev_normal(shape, tid, std=1.0, dtype=None):
    from synth import device as sd
    t = torch.empty(shape, dtype=dtype or torch.bfloat16, device="cuda")
    sd.fill_tensor_normal(t, SEED, tid, std)
    return t


def _host_rows(tid, ncols, rows, std=1.0, bf16=True):
    f = synth.normal_bf16_as_f32 if bf16 else synth.normal_f32
    return np.stack([f(SEED, tid, (ncols,), std, start=int(r) * ncols) for r in rows]).astype(np.float64)


def _bf16(t):
    return t.float().cpu().numpy().astype(np.float64)


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("name,M,N,K,epi,split", [
    ("qkv", 32768, QKV, C, 0, False), ("o", 32768, C, HQ * D, 0, False), ("gate_up", 32768, 2 * F, C, 3, False),
    ("down", 32768, C, F, 0, False), ("head_last_rows", 32, V, C, 1, True), ("head_all_rows", 2048, V, C, 1, False),
    ("decode_gate_up", 32, 2 * F, C, 3, True), ("decode_down", 32, C, F, 0, True),
    ("decode_o", 32, C, HQ * D, 0, True), ("decode_qkv_m7", 7, QKV, C, 0, True),
    ("decode_down_nosplit", 32, C, F, 0, False), ("decode_gate_up_m1_nosplit", 1, 2 * F, C, 3, False),
    # two blocks of 32 token rows against one weight read (two cohorts of a pipelined decode)
    ("decode64_gate_up", 64, 2 * F, C, 3, True), ("decode64_o", 64, C, HQ * D, 0, True),
    ("decode64_down_m45", 45, C, F, 0, True), ("head64_rows", 64, V, C, 1, True),
    ("decode64_qkv_nosplit_m33", 33, QKV, C, 0, False),
    # row counts that end inside a 256-row tile (the epilogue's row bound)
    ("gate_up_rows1000", 1000, 2 * F, C, 3, False), ("head_rows300", 300, V, C, 1, False),
    # K % 64 == 32: the 32-deep eight-wave kernel
    ("qkv_k4064_rows4133", 4133, QKV, 4064, 0, False), ("gate_up_k4064_rows1000", 1000, 2 * 2048, 4064, 3, False),
])
def test_gemm_full_size_sampled(name, M, N, K, epi, split):
    """9B-shape projections; M <= 64 is the decode kernel, with K split over
    workgroups (scratch given) or one workgroup per weight tile."""
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    print(f"gemm {name} M={M} N={N} K={K} split={split}", flush=True)
    a = _dev_normal((M, K), 11)
    b = _dev_normal((N, K), 12, 0.02)
    ncol = N // 2 if epi == 3 else N
    c = torch.empty(M, ncol, dtype=torch.float32 if epi == 1 else torch.bfloat16, device="cuda")
    Fa = N // 2 if epi == 3 else 0
    nbytes = A.loop_op_gemm_bytes(A.LOOP_BF16, epi, M, N, K, Fa) if split else 0
    if split and name.startswith("decode"):
        assert nbytes > 0          # these shapes do split on a 256-CU device
    scr = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    for _ in range(2):             # the second call runs on the counters the first one left
        A.loop_op_gemm(A.LOOP_BF16, epi, M, N, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), ncol, Fa,
                       _stream(), scr.data_ptr() if nbytes else None, nbytes)
    torch.cuda.synchronize()
    rng = np.random.default_rng(hash(name) & 0xFFFF)
    rows = np.unique(np.concatenate([rng.integers(0, M, 24), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, ncol, 24), [0, ncol - 1]]))
    Ar = _host_rows(11, K, rows)
    got = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].float().cpu().numpy()
    if epi == 3:
        Bg = _host_rows(12, K, cols, 0.02)
        Bu = _host_rows(12, K, cols + ncol, 0.02)
        g, u = Ar @ Bg.T, Ar @ Bu.T
        ref = g / (1 + np.exp(-g)) * u
        scale = (np.abs(Ar) @ np.abs(Bg).T) * np.abs(u) + (np.abs(Ar) @ np.abs(Bu).T) * np.abs(g) + 1e-30
        bound = 2.0 ** -8 * np.abs(ref) + 2e-5 * scale
    else:
        Br = _host_rows(12, K, cols, 0.02)
        ref = Ar @ Br.T
        scale = np.abs(Ar) @ np.abs(Br).T
        bound = 1e-5 * scale + (2.0 ** -8 * np.abs(ref) if epi == 0 else 0.0)
    assert np.all(np.abs(got - ref) <= bound), float((np.abs(got - ref) / bound).max())


# ------------------------------------------------------------------ mHC
def test_mhc_isolated_full_size_sampled():
    """2 streams x 4096 bf16 for 65,536 tokens, per-token map logits N(0, 1)
    (maps from the oracle's definition), layer output y ~ N(0, 1)."""
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    T = 65536
    X = _dev_normal((T, 2, C), 21)
    X0 = X.clone()
    y = _dev_normal((T, C), 22)
    logits_in = synth.normal_f32(SEED, 23, (T, 8))
    pre_i = 1 / (1 + np.exp(-logits_in[:, 0:2].astype(np.float64)))
    post_i = 2 / (1 + np.exp(-logits_in[:, 2:4].astype(np.float64)))
    R = logits_in[:, 4:8].astype(np.float64).reshape(T, 2, 2)
    res_i = M.sinkhorn(np.exp(R - R.max(axis=(1, 2), keepdims=True)), 20)
    maps_in = np.concatenate([pre_i, post_i, res_i.reshape(T, 4)], 1).astype(np.float32)
    mi = torch.from_numpy(maps_in).cuda()
    mo = torch.empty(T, 8, dtype=torch.float32, device="cuda")
    w = _dev_normal((8, 2 * C), 24, 0.02, torch.float32)
    bb = _dev_normal((8,), 25, 0.02, torch.float32)
    gamma = torch.ones(C, dtype=torch.float32, device="cuda")
    u = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    nb = A.loop_op_mhc_bytes(C)
    scr = torch.empty(nb, dtype=torch.uint8, device="cuda")
    A.loop_op_mhc(A.LOOP_BF16, A.LOOP_MHC_MID, T, C, 20, 1e-6, y.data_ptr(), None, X.data_ptr(), mi.data_ptr(),
                  mo.data_ptr(), w.data_ptr(), bb.data_ptr(), gamma.data_ptr(), u.data_ptr(), scr.data_ptr(), nb,
                  _stream())
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([rng.integers(0, T, 48), [0, T - 1]]))
    tt = torch.from_numpy(toks).cuda()
    x_old = _bf16(X0[tt])
    y_h = _bf16(y[tt])
    W = w.cpu().numpy().astype(np.float64)
    Bv = bb.cpu().numpy().astype(np.float64)
    mi_s = maps_in[toks].astype(np.float64)
    Xn = M.round_bf16(np.einsum("tij,tjc->tic", mi_s[:, 4:8].reshape(-1, 2, 2), x_old)
                      + mi_s[:, 2:4, None] * y_h[:, None, :])
    pre, post, res, _ = M.mhc_maps(Xn, W, Bv, 20, 1e-6)
    x_in = pre[:, 0:1] * Xn[:, 0] + pre[:, 1:2] * Xn[:, 1]
    u_ref = M.rmsnorm(x_in, np.ones(C), 1e-6)
    gX = _bf16(X[tt])
    # Both sides round once to bf16 and may land one ulp (<= 2^-7 |x|) apart;
    # when the three terms cancel, the float32 sum itself carries an error of
    # a few float32 ulps of the largest term.
    terms = (np.abs(mi_s[:, 4:8].reshape(-1, 2, 2)) @ np.abs(x_old)) + np.abs(mi_s[:, 2:4, None] * y_h[:, None, :])
    bound = 2.0 ** -7 * np.abs(Xn) + 4 * 2.0 ** -24 * terms
    print("mhc X' worst diff / bound:", float((np.abs(gX - Xn) / bound).max()),
          "flips:", int((gX != Xn).sum()), flush=True)
    assert np.all(np.abs(gX - Xn) <= bound)
    gm = mo[tt].cpu().numpy().astype(np.float64)
    ref_maps = np.concatenate([pre, post, res.reshape(-1, 4)], 1)
    assert np.abs(gm - ref_maps).max() < 1e-4      # maps of the host's X' (X' may differ by one-ulp roundings)
    # Maps of the X' the kernel wrote, against the float64 definition: W is
    # carried in three bf16 parts (within 2^-27 of float32 W) and X' is bf16,
    # so the projection is float32-exact products with float32 sums of 8192
    # terms; the logits then carry a few float32 ulps of sum |W x_hat|
    # (about 1e-6 here), and the maps less.  A W held to 16 bits would miss
    # this by an order of magnitude.
    pre_g, post_g, res_g, _ = M.mhc_maps(gX, W, Bv, 20, 1e-6)
    ref_own = np.concatenate([pre_g, post_g, res_g.reshape(-1, 4)], 1)
    print("mhc maps: max |diff| against the maps of the kernel's own X':", float(np.abs(gm - ref_own).max()),
          flush=True)
    assert np.abs(gm - ref_own).max() < 2e-6
    assert np.abs(gm[:, 4:8].reshape(-1, 2, 2).sum(1) - 1).max() < 1e-5     # columns
    gu = _bf16(u[tt])
    assert np.all(np.abs(gu - u_ref) <= 2.0 ** -6 * np.abs(u_ref) + 1e-3)


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_full_attention_prefill_full_size_sampled(layout):
    """One full-attention execution of the 32K prefill: B=1, S=32768, 32 q / 8 kv heads of 128 or 16 / 4 of 256."""
    HQ, HKV, D, QKV = _lay(layout)
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    S = 32768
    q = _dev_normal((S, QKV), 31)            # q columns of the QKV output row
    k = _dev_normal((1, HKV, S, D), 32)
    vt = torch.empty(1, HKV, D, S, dtype=torch.bfloat16, device="cuda")
    from synth import device as sd
    sd.fill_normal4(vt.data_ptr(), True, (1, HKV, S, D), (HKV * D * S, D * S, 1, S), SEED, 33, 1.0,
                    stream=_stream())
    out = torch.empty(S, HQ * D, dtype=torch.bfloat16, device="cuda")
    A.loop_op_attention(A.LOOP_BF16, 1, S, 0, S, HQ, HKV, D, q.data_ptr(), QKV, k.data_ptr(), vt.data_ptr(),
                        out.data_ptr(), HQ * D, _stream())
    torch.cuda.synchronize()
    for pos, head in [(0, 0), (31, 5), (4095, 13), (20000, 30), (S - 1, 31), (S - 1, 2)]:
        head %= HQ
        kvh = head // (HQ // HKV)
        qr = synth.normal_bf16_as_f32(SEED, 31, (QKV,), start=pos * QKV)[head * D:(head + 1) * D]
        K = synth.normal_bf16_as_f32(SEED, 32, (pos + 1, D), start=(kvh * S) * D)
        Vv = synth.normal_bf16_as_f32(SEED, 33, (pos + 1, D), start=(kvh * S) * D)
        ref = M.full_attention(qr[None, None, None, :], K[None, :, None, :], Vv[None, :, None, :], pos)[0, 0, 0]
        got = out[pos, head * D:(head + 1) * D].float().cpu().numpy()
        err = np.abs(got - ref).max() / np.abs(ref).max()
        print("attn", pos, head, err, flush=True)
        assert err < 2e-2


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_full_attention_chunk_continuation_sampled(layout):
    """A prefill chunk that continues a long cache (chunked prefill): 700 new
    positions at pos0 = 30000 (not a tile multiple) over S_max = 30720, B=2."""
    HQ, HKV, D, QKV = _lay(layout)
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    from synth import device as sd
    B, pos0, S = 2, 30000, 700
    L = pos0 + S
    Smax = (L + 63) // 64 * 64
    q = _dev_normal((B * S, QKV), 34)
    kc = torch.empty(B, HKV, Smax, D, dtype=torch.bfloat16, device="cuda")
    vt = torch.empty(B, HKV, D, Smax, dtype=torch.bfloat16, device="cuda")
    sd.fill_tensor_normal(kc, SEED, 99, 1.0)          # arbitrary values past the end
    sd.fill_tensor_normal(vt, SEED, 98, 1.0)
    sd.fill_normal4(kc.data_ptr(), True, (B, HKV, L, D), (HKV * Smax * D, Smax * D, D, 1), SEED, 35, 1.0,
                    stream=_stream())
    sd.fill_normal4(vt.data_ptr(), True, (B, HKV, L, D), (HKV * D * Smax, D * Smax, 1, Smax), SEED, 36, 1.0,
                    stream=_stream())
    out = torch.empty(B * S, HQ * D, dtype=torch.bfloat16, device="cuda")
    A.loop_op_attention(A.LOOP_BF16, B, S, pos0, Smax, HQ, HKV, D, q.data_ptr(), QKV, kc.data_ptr(), vt.data_ptr(),
                        out.data_ptr(), HQ * D, _stream())
    torch.cuda.synchronize()
    for b, t, head in [(0, 0, 0), (0, 63, 7), (1, 64, 12), (1, 699, 31), (0, 350, 20)]:
        head %= HQ
        kvh = head // (HQ // HKV)
        row = b * S + t
        qr = synth.normal_bf16_as_f32(SEED, 34, (QKV,), start=row * QKV)[head * D:(head + 1) * D]
        base = ((b * HKV + kvh) * L) * D
        K = synth.normal_bf16_as_f32(SEED, 35, (pos0 + t + 1, D), start=base)
        Vv = synth.normal_bf16_as_f32(SEED, 36, (pos0 + t + 1, D), start=base)
        ref = M.full_attention(qr[None, None, None, :], K[None, :, None, :], Vv[None, :, None, :], pos0 + t)[0, 0, 0]
        got = out[row, head * D:(head + 1) * D].float().cpu().numpy()
        err = np.abs(got - ref).max() / np.abs(ref).max()
        print("attn chunk", b, t, head, err, flush=True)
        assert err < 2e-2


@pytest.mark.parametrize("B,ctx,samples", [
    (32, 32768, [(0, 0), (7, 9), (31, 31), (16, 4)]),     # one split per (sequence, KV head)
    (2, 5001, [(0, 0), (1, 13), (1, 31)]),                # several splits, ragged last split
    (1, 37, [(0, 0), (0, 30)]),                           # fewer keys than one round
])
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_decode_attention_full_size_sampled(B, ctx, samples, layout):
    """B sequences of ctx cached positions + 1 new, 8 KV heads of 128 or 4 of 256."""
    HQ, HKV, D, QKV = _lay(layout)
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    from synth import device as sd
    print(f"decode attention B={B} ctx={ctx}", flush=True)
    Smax = (ctx + 1 + 63) // 64 * 64
    kc = torch.zeros(B, HKV, Smax, D, dtype=torch.bfloat16, device="cuda")
    vt = torch.zeros(B, HKV, D, Smax, dtype=torch.bfloat16, device="cuda")
    L = ctx + 1
    sd.fill_normal4(kc.data_ptr(), True, (B, HKV, L, D), (HKV * Smax * D, Smax * D, D, 1), SEED, 41, 1.0,
                    stream=_stream())
    sd.fill_normal4(vt.data_ptr(), True, (B, HKV, L, D), (HKV * D * Smax, D * Smax, 1, Smax), SEED, 42, 1.0,
                    stream=_stream())
    q = _dev_normal((B, QKV), 43)
    out = torch.empty(B, HQ * D, dtype=torch.bfloat16, device="cuda")
    nb = A.loop_op_attention_decode_bytes(B, 1, HQ, D, Smax)
    scr = torch.empty(nb, dtype=torch.uint8, device="cuda")
    A.loop_op_attention_decode(A.LOOP_BF16, B, 1, ctx, Smax, HQ, HKV, D, q.data_ptr(), QKV, kc.data_ptr(),
                               vt.data_ptr(), out.data_ptr(), HQ * D, scr.data_ptr(), nb, _stream())
    torch.cuda.synchronize()
    for b, head in samples:
        head %= HQ
        kvh = head // (HQ // HKV)
        qr = synth.normal_bf16_as_f32(SEED, 43, (QKV,), start=b * QKV)[head * D:(head + 1) * D]
        base = ((b * HKV + kvh) * L) * D
        K = synth.normal_bf16_as_f32(SEED, 41, (L, D), start=base)
        Vv = synth.normal_bf16_as_f32(SEED, 42, (L, D), start=base)
        ref = M.full_attention(qr[None, None, None, :], K[None, :, None, :], Vv[None, :, None, :], ctx)[0, 0, 0]
        got = out[b, head * D:(head + 1) * D].float().cpu().numpy()
        err = np.abs(got - ref).max() / np.abs(ref).max()
        print("decode attn", b, head, err, flush=True)
        assert err < 2e-2


@pytest.mark.parametrize("pos,samples", [
    # 32 sequences from 1 to 32,768 keys: pieces span several short sequences
    ([32767, 0, 63, 64, 65, 1, 31000, 12345] + [(b * 7919) % 32768 for b in range(8, 32)],
     [(0, 0), (1, 5), (2, 31), (3, 8), (4, 17), (5, 2), (6, 30), (9, 12), (31, 7)]),
    ([5000, 3], [(0, 0), (0, 22), (1, 0), (1, 31)]),
])
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_decode_attention_stream_k_full_size_sampled(pos, samples, layout):
    """The stream-K split of the ragged decode (sequences' keys laid end to end
    and cut into equal pieces per KV head, partials merged per row) at the 9B
    layouts: sequence b attends to its own pos[b] + 1 keys; slots hold NaN past
    each sequence's keys."""
    HQ, HKV, D, QKV = _lay(layout)
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    from synth import device as sd
    B, mx = len(pos), max(pos)
    print(f"stream-K decode attention B={B} max start {mx}", flush=True)
    Smax = (mx + 1 + 63) // 64 * 64
    L = mx + 1
    kc = torch.zeros(B, HKV, Smax, D, dtype=torch.bfloat16, device="cuda")
    vt = torch.zeros(B, HKV, D, Smax, dtype=torch.bfloat16, device="cuda")
    sd.fill_normal4(kc.data_ptr(), True, (B, HKV, L, D), (HKV * Smax * D, Smax * D, D, 1), SEED, 51, 1.0,
                    stream=_stream())
    sd.fill_normal4(vt.data_ptr(), True, (B, HKV, L, D), (HKV * D * Smax, D * Smax, 1, Smax), SEED, 52, 1.0,
                    stream=_stream())
    for b, p in enumerate(pos):
        kc[b, :, p + 1:, :] = float("nan")
        vt[b, :, :, p + 1:] = float("nan")
    q = _dev_normal((B, QKV), 53)
    starts = np.array(pos, np.int32)
    out = torch.empty(B, HQ * D, dtype=torch.bfloat16, device="cuda")
    nb = A.loop_op_attention_decode_stream_k_bytes(B, 1, HQ, HKV, D)
    scr = torch.empty(nb, dtype=torch.uint8, device="cuda")
    A.loop_op_attention_decode_stream_k(A.LOOP_BF16, B, 1, starts.ctypes.data, Smax, HQ, HKV, D, q.data_ptr(), QKV,
                                        kc.data_ptr(), vt.data_ptr(), out.data_ptr(), HQ * D, scr.data_ptr(), nb,
                                        _stream())
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all().item()
    for b, head in samples:
        head %= HQ
        kvh = head // (HQ // HKV)
        n = pos[b] + 1
        qr = synth.normal_bf16_as_f32(SEED, 53, (QKV,), start=b * QKV)[head * D:(head + 1) * D]
        base = ((b * HKV + kvh) * L) * D
        K = synth.normal_bf16_as_f32(SEED, 51, (n, D), start=base)
        Vv = synth.normal_bf16_as_f32(SEED, 52, (n, D), start=base)
        ref = M.full_attention(qr[None, None, None, :], K[None, :, None, :], Vv[None, :, None, :], pos[b])[0, 0, 0]
        got = out[b, head * D:(head + 1) * D].float().cpu().numpy()
        err = np.abs(got - ref).max() / np.abs(ref).max()
        print("stream-K decode attn", b, pos[b], head, err, flush=True)
        assert err < 2e-2


@pytest.mark.parametrize("pos,samples", [
    # 32 sequences of the decode batch at lengths up to the 32K context: one split each
    ([32767, 0, 63, 64, 65, 1, 31000, 12345] + [(b * 7919) % 32768 for b in range(8, 32)],
     [(0, 0), (1, 5), (2, 31), (3, 8), (4, 17), (5, 2), (6, 30), (9, 12)]),
    # two sequences: the short one has keys in the first of many splits only
    ([5000, 3], [(0, 0), (0, 22), (1, 0), (1, 31)]),
])
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_decode_attention_ragged_full_size_sampled(pos, samples, layout):
    """Sequence b attends to its own pos[b] + 1 keys; slots hold NaN past
    each sequence's keys, which the kernel must neither weigh nor multiply."""
    HQ, HKV, D, QKV = _lay(layout)
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    from synth import device as sd
    B, mx = len(pos), max(pos)
    print(f"ragged decode attention B={B} max start {mx}", flush=True)
    Smax = (mx + 1 + 63) // 64 * 64
    L = mx + 1
    kc = torch.zeros(B, HKV, Smax, D, dtype=torch.bfloat16, device="cuda")
    vt = torch.zeros(B, HKV, D, Smax, dtype=torch.bfloat16, device="cuda")
    sd.fill_normal4(kc.data_ptr(), True, (B, HKV, L, D), (HKV * Smax * D, Smax * D, D, 1), SEED, 51, 1.0,
                    stream=_stream())
    sd.fill_normal4(vt.data_ptr(), True, (B, HKV, L, D), (HKV * D * Smax, D * Smax, 1, Smax), SEED, 52, 1.0,
                    stream=_stream())
    for b, p in enumerate(pos):
        kc[b, :, p + 1:, :] = float("nan")
        vt[b, :, :, p + 1:] = float("nan")
    q = _dev_normal((B, QKV), 53)
    pos_dev = torch.tensor(pos, dtype=torch.int32, device="cuda")
    out = torch.empty(B, HQ * D, dtype=torch.bfloat16, device="cuda")
    nb = A.loop_op_attention_decode_bytes(B, 1, HQ, D, Smax)
    scr = torch.empty(nb, dtype=torch.uint8, device="cuda")
    A.loop_op_attention_decode_ragged(A.LOOP_BF16, B, 1, pos_dev.data_ptr(), mx, Smax, HQ, HKV, D, q.data_ptr(), QKV,
                                      kc.data_ptr(), vt.data_ptr(), out.data_ptr(), HQ * D, scr.data_ptr(), nb,
                                      _stream())
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all().item()
    for b, head in samples:
        head %= HQ
        kvh = head // (HQ // HKV)
        n = pos[b] + 1
        qr = synth.normal_bf16_as_f32(SEED, 53, (QKV,), start=b * QKV)[head * D:(head + 1) * D]
        base = ((b * HKV + kvh) * L) * D
        K = synth.normal_bf16_as_f32(SEED, 51, (n, D), start=base)
        Vv = synth.normal_bf16_as_f32(SEED, 52, (n, D), start=base)
        ref = M.full_attention(qr[None, None, None, :], K[None, :, None, :], Vv[None, :, None, :], pos[b])[0, 0, 0]
        got = out[b, head * D:(head + 1) * D].float().cpu().numpy()
        err = np.abs(got - ref).max() / np.abs(ref).max()
        print("ragged decode attn", b, pos[b], head, err, flush=True)
        assert err < 2e-2


# ------------------------------------------------------------------ linear attention
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_linear_attention_chunked_full_size_sampled(layout):
    """One linear-attention execution of the 32K prefill, fresh state: outputs
    of one KV group at sampled positions, and the final state of that group,
    against the oracle's recurrence."""
    HQ, HKV, D, QKV = _lay(layout)
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    S = 32768
    qkv = _dev_normal((S, QKV), 51)
    out = torch.empty(S, HQ * D, dtype=torch.bfloat16, device="cuda")
    St = torch.zeros(HKV, D, D, dtype=torch.float32, device="cuda")
    zt = torch.zeros(HKV, D, dtype=torch.float32, device="cuda")
    nb = A.loop_op_linear_bytes(1, S, HKV, D)
    scr = torch.empty(nb, dtype=torch.uint8, device="cuda")
    A.loop_op_linear(A.LOOP_BF16, 1, 1, S, HQ, HKV, D, 1e-6, qkv.data_ptr(), QKV, St.data_ptr(), zt.data_ptr(), 1,
                     out.data_ptr(), HQ * D, scr.data_ptr(), nb, _stream())
    torch.cuda.synchronize()
    kvh = 5 % HKV
    G = HQ // HKV
    heads = list(range(kvh * G, kvh * G + G))
    rows = synth.normal_bf16_as_f32(SEED, 51, (S, QKV))
    q = rows[:, [h * D + i for h in heads for i in range(D)]].reshape(1, S, G, D)
    k = rows[:, (HQ + kvh) * D:(HQ + kvh + 1) * D].reshape(1, S, 1, D)
    v = rows[:, (HQ + HKV + kvh) * D:(HQ + HKV + kvh + 1) * D].reshape(1, S, 1, D)
    del rows
    sample = [0, 1, 63, 64, 65, 1000, 4097, 16383, 20000, S - 1]
    o, Sf, zf = M.linear_attention(q, k, v, np.zeros((1, 1, D, D)), np.zeros((1, 1, D)), 1e-6)
    for t in sample:
        for hi, h in enumerate(heads):
            got = out[t, h * D:(h + 1) * D].float().cpu().numpy()
            ref = o[0, t, hi]
            assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max(), (t, h)
    gS = St[kvh].cpu().numpy()
    assert np.abs(gS - Sf[0, 0]).max() <= 1e-4 * np.abs(Sf[0, 0]).max()
    assert np.abs(zt[kvh].cpu().numpy() - zf[0, 0]).max() <= 1e-4 * np.abs(zf[0, 0]).max()


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_linear_attention_decode_prefilled_state(layout):
    """B=32 decode with pre-filled states S ~ N(0, 1), z = |N(0, 1)| (all outputs)."""
    HQ, HKV, D, QKV = _lay(layout)
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    B = 32
    qkv = _dev_normal((B, QKV), 61)
    S0 = _dev_normal((B, HKV, D, D), 62, 1.0, torch.float32)
    from synth import device as sd
    z0 = torch.empty(B, HKV, D, dtype=torch.float32, device="cuda")
    sd.fill_tensor_normal(z0, SEED, 63, 1.0, absval=True)
    S_host = S0.cpu().numpy().astype(np.float64)
    z_host = z0.cpu().numpy().astype(np.float64)
    out = torch.empty(B, HQ * D, dtype=torch.bfloat16, device="cuda")
    A.loop_op_linear(A.LOOP_BF16, 0, B, 1, HQ, HKV, D, 1e-6, qkv.data_ptr(), QKV, S0.data_ptr(), z0.data_ptr(), 0,
                     out.data_ptr(), HQ * D, None, 0, _stream())
    torch.cuda.synchronize()
    rows = synth.normal_bf16_as_f32(SEED, 61, (B, QKV))
    q = rows[:, :HQ * D].reshape(B, 1, HQ, D)
    k = rows[:, HQ * D:(HQ + HKV) * D].reshape(B, 1, HKV, D)
    v = rows[:, (HQ + HKV) * D:].reshape(B, 1, HKV, D)
    o, Sf, zf = M.linear_attention(q, k, v, S_host, z_host, 1e-6)
    got = out.float().cpu().numpy().reshape(B, HQ, D)
    ref = o[:, 0]
    # the denominator of a pre-filled state can be small: compare per row
    err = np.abs(got - ref).max(-1) / np.abs(ref).max(-1)
    assert err.max() < 2e-2, err.max()
    assert np.abs(S0.cpu().numpy() - Sf).max() <= 1e-5 * np.abs(Sf).max()


@pytest.mark.parametrize("Cn", [256, 512])
def test_mhc_narrow_streams(Cn):
    """The mHC site on narrow streams (512 tokens): at C = 512 the tiled MFMA
    path, at C = 256 the per-token path (a wave's C / 8 = 32 channels are one
    32-channel step, less than the tiled path's two-step load group).  Maps
    of the kernel's own X' against the float64 definition, X' and u."""
    need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    T = 512
    X = _dev_normal((T, 2, Cn), 71)
    X0 = X.clone()
    y = _dev_normal((T, Cn), 72)
    logits_in = synth.normal_f32(SEED, 73, (T, 8))
    pre_i = 1 / (1 + np.exp(-logits_in[:, 0:2].astype(np.float64)))
    post_i = 2 / (1 + np.exp(-logits_in[:, 2:4].astype(np.float64)))
    R = logits_in[:, 4:8].astype(np.float64).reshape(T, 2, 2)
    res_i = M.sinkhorn(np.exp(R - R.max(axis=(1, 2), keepdims=True)), 20)
    maps_in = np.concatenate([pre_i, post_i, res_i.reshape(T, 4)], 1).astype(np.float32)
    mi = torch.from_numpy(maps_in).cuda()
    mo = torch.empty(T, 8, dtype=torch.float32, device="cuda")
    w = _dev_normal((8, 2 * Cn), 74, 0.02, torch.float32)
    bb = _dev_normal((8,), 75, 0.02, torch.float32)
    gamma = torch.ones(Cn, dtype=torch.float32, device="cuda")
    u = torch.empty(T, Cn, dtype=torch.bfloat16, device="cuda")
    nb = A.loop_op_mhc_bytes(Cn)
    scr = torch.empty(nb, dtype=torch.uint8, device="cuda")
    A.loop_op_mhc(A.LOOP_BF16, A.LOOP_MHC_MID, T, Cn, 20, 1e-6, y.data_ptr(), None, X.data_ptr(), mi.data_ptr(),
                  mo.data_ptr(), w.data_ptr(), bb.data_ptr(), gamma.data_ptr(), u.data_ptr(), scr.data_ptr(), nb,
                  _stream())
    torch.cuda.synchronize()
    x_old, y_h, gX = _bf16(X0), _bf16(y), _bf16(X)
    mi_s = maps_in.astype(np.float64)
    Xn = M.round_bf16(np.einsum("tij,tjc->tic", mi_s[:, 4:8].reshape(-1, 2, 2), x_old)
                      + mi_s[:, 2:4, None] * y_h[:, None, :])
    terms = (np.abs(mi_s[:, 4:8].reshape(-1, 2, 2)) @ np.abs(x_old)) + np.abs(mi_s[:, 2:4, None] * y_h[:, None, :])
    assert np.all(np.abs(gX - Xn) <= 2.0 ** -7 * np.abs(Xn) + 4 * 2.0 ** -24 * terms)
    W, Bv = w.cpu().numpy().astype(np.float64), bb.cpu().numpy().astype(np.float64)
    pre, post, res, _ = M.mhc_maps(gX, W, Bv, 20, 1e-6)
    ref = np.concatenate([pre, post, res.reshape(-1, 4)], 1)
    err = float(np.abs(mo.cpu().numpy().astype(np.float64) - ref).max())
    print(f"mhc C={Cn}: maps max |diff| {err:.2e}", flush=True)
    assert err < 2e-6
    u_ref = M.rmsnorm(pre[:, 0:1] * gX[:, 0] + pre[:, 1:2] * gX[:, 1], np.ones(Cn), 1e-6)
    assert np.all(np.abs(_bf16(u) - u_ref) <= 2.0 ** -6 * np.abs(u_ref) + 1e-3)
