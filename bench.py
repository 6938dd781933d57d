"""Throughput of the looped decoder forward pass on one MI355X.

A step is one prefill of the Loop-9B-shaped model (32 stored layers, block
[4, 28) run twice: 56 layer executions; hidden 4096, FFN 12288, 32 q / 8 kv
heads of 128, vocabulary 248,320) over B=1, S=32,768 synthetic token ids,
through every step of the path (embed, 56 executions with two-stream mHC,
linear and full attention, SwiGLU, final norm, head on the last position).
The same run also times a decode step of B=32 sequences holding 32,768
pre-filled positions each, the dominant kernel on its own (HIP events on the
stream it runs on), and the CPU oracle on a bounded sample.

Prints ONE JSON line.  Inputs and weights are synthetic random-init values
already resident in HBM when a timed region starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "looped-decoder tokens/sec (56 layer execs, 9B shape): prefill + decode; % roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc runs
# of `bench.py --profile dominant` (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), each scaled by the same counter's reading for a plain 1 GiB
# device copy in that run.  Valid only for the kernel source it was taken on:
# the hash of k_gemm.hip + common.h must match, else traffic is reported null.
DOMINANT_COUNTERS = {"source_sha256_16": "010e5bf362528ce1", "fetch_kib": 4748225.5, "write_kib": 786432.0,
                     "copy_fetch_kib": 524308.2, "copy_write_kib": 1048576.0}

NINE_B = dict(vocab=248320, hidden=4096, ffn=12288, n_heads=32, n_kv_heads=8, head_dim=128,
              n_layers=32, loop_start=4, loop_end=28, n_passes=2, dtype="bf16")
# the same model with the attention heads one page gives (16 query / 4 KV heads
# of 256: "How Does SenseNova-Loop Get More Depth Without More Parameters?",
# section on the hybrid attention pattern); equal projection sizes
NINE_B_D256 = dict(NINE_B, n_heads=16, n_kv_heads=4, head_dim=256)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_hash():
    """Hash of the GEMM sources with comments and blank space removed, so that
    a change of comments alone keeps the measured counters valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("k_gemm.hip", "common.h"):
        with open(os.path.join(ROOT, "looped_weight_shared_loop_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def dominant_traffic():
    """Measured HBM bytes per launch of the dominant kernel, or None when the
    kernel source differs from the one the counters were read on."""
    c = DOMINANT_COUNTERS
    if gemm_source_hash() != c["source_sha256_16"]:
        return None
    fetch = c["fetch_kib"] * 1024 * ((1 << 30) / (c["copy_fetch_kib"] * 1024))
    write = c["write_kib"] * 1024 * ((1 << 30) / (c["copy_write_kib"] * 1024))
    return fetch + write


def prefill_flops(cfg, S, B=1):
    """Algorithmic FLOPs of one prefill: 2 * params * tokens for every GEMM
    execution, 2 S^2 d Hq per causal full-attention execution (QK^T and PV,
    causal half), the recurrent linear-attention cost (per token per
    execution: S update 2 d^2 Hkv, readout 2 d^2 Hq, normaliser ~2 d (Hq+Hkv)),
    and the head on the emitted rows."""
    C, F, d, Hq, Hkv = cfg["hidden"], cfg["ffn"], cfg["head_dim"], cfg["n_heads"], cfg["n_kv_heads"]
    per_layer = (Hq + 2 * Hkv) * d * C + C * Hq * d + 2 * F * C + C * F
    n_exec = cfg["loop_start"] + cfg["n_passes"] * (cfg["loop_end"] - cfg["loop_start"]) + \
        (cfg["n_layers"] - cfg["loop_end"])
    n_full = 0
    for i in list(range(cfg["loop_start"])) + list(range(cfg["loop_start"], cfg["loop_end"])) * cfg["n_passes"] + \
            list(range(cfg["loop_end"], cfg["n_layers"])):
        n_full += (i % 4 == 3)
    T = B * S
    gemm = 2.0 * per_layer * T * n_exec
    attn = n_full * B * 2.0 * S * S * d * Hq
    lin = (n_exec - n_full) * T * (2.0 * d * d * Hkv + 2.0 * d * d * Hq + 2.0 * d * (Hq + Hkv))
    head = 2.0 * cfg["vocab"] * C * B
    return gemm + attn + lin + head, gemm, attn, lin


def decode_pipelined_bytes(cfg, B, ctx):
    """Bytes one pass-pipelined call must move (B tokens leave per call): every
    stored layer's weights once (the looped block serves all cohorts), the
    head, and the same KV and linear-state traffic as a B-token decode step."""
    tot, w, kv, lin = decode_bytes(cfg, B, ctx)
    C, F, d, Hq, Hkv = cfg["hidden"], cfg["ffn"], cfg["head_dim"], cfg["n_heads"], cfg["n_kv_heads"]
    per_layer = ((Hq + 2 * Hkv) * d * C + C * Hq * d + 2 * F * C + C * F) * 2
    w1 = per_layer * cfg["n_layers"] + cfg["vocab"] * C * 2
    return w1 + kv + lin, w1, kv, lin


def decode_bytes(cfg, B, ctx):
    """Bytes one decode step must move: every layer execution's weights (the
    shared block twice), the head, every KV cache (K and V of `ctx` positions),
    every linear state read and written."""
    C, F, d, Hq, Hkv, V = cfg["hidden"], cfg["ffn"], cfg["head_dim"], cfg["n_heads"], cfg["n_kv_heads"], cfg["vocab"]
    per_layer = ((Hq + 2 * Hkv) * d * C + C * Hq * d + 2 * F * C + C * F) * 2
    n_exec, n_full = 56, 14
    w = per_layer * n_exec + V * C * 2
    kv = n_full * B * Hkv * ctx * d * 2 * 2
    lin = (n_exec - n_full) * B * Hkv * (d * d + d) * 4 * 2
    return w + kv + lin, w, kv, lin


def time_prefill(L, torch, model, S, steps, warmup):
    import synth
    from synth import device as sd
    st = model.new_state(1, S)
    toks = torch.empty(1, S, dtype=torch.int32, device="cuda")
    sd.fill_tensor_uniform_int(toks, 1, synth.TID_TOKENS, model.cfg.vocab)
    model.workspace(1, S, S)
    for i in range(warmup):
        model.prefill(st, toks)
        torch.cuda.synchronize()
        log(f"prefill warmup {i + 1}/{warmup} done")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        out = model.prefill(st, toks)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    log(f"prefill: {ms:.1f} ms/step (events), wall {wall / steps * 1e3:.1f} ms/step")
    st.check()
    assert torch.isfinite(out).all().item()
    st.close()
    return ms


def time_long_prefill(L, torch, model, S_long, chunk):
    """Chunked prefill of one sequence of S_long positions in chunks of `chunk`
    (LOOP_CONTINUE), every chunk through all 56 executions; one timed pass."""
    import synth
    from synth import device as sd
    st = model.new_state(1, S_long)
    toks = torch.empty(1, S_long, dtype=torch.int32, device="cuda")
    sd.fill_tensor_uniform_int(toks, 1, synth.TID_TOKENS + 200, model.cfg.vocab)
    model.workspace(1, chunk, S_long)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for c in range(S_long // chunk):
        out = model.prefill(st, toks[:, c * chunk:(c + 1) * chunk], cont=c > 0)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    st.check()
    assert torch.isfinite(out).all().item()
    log(f"chunked prefill S={S_long} (chunks of {chunk}): {ms:.1f} ms")
    st.close()
    return ms


def time_dominant_gemm(L, torch, S, iters=10):
    """The SwiGLU gate/up projection at the prefill shape: M = 32768 tokens,
    N = 2 x 12288 weight rows, K = 4096 (the largest GEMM, 44% of the FLOPs)."""
    from looped_weight_shared_loop_amd import _abi as A
    from synth import device as sd
    M, F, K = S, NINE_B["ffn"], NINE_B["hidden"]
    a = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    b = torch.empty(2 * F, K, dtype=torch.bfloat16, device="cuda")
    c = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
    sd.fill_tensor_normal(a, 3, 1, 1.0)
    sd.fill_tensor_normal(b, 3, 2, 0.02)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        A.loop_op_gemm(A.LOOP_BF16, A.LOOP_EPI_SWIGLU, M, 2 * F, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(),
                       F, F, stream, None, 0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        A.loop_op_gemm(A.LOOP_BF16, A.LOOP_EPI_SWIGLU, M, 2 * F, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(),
                       F, F, stream, None, 0)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    flops = 2.0 * M * 2 * F * K
    log(f"gate/up GEMM: {ms:.3f} ms/launch, {flops / ms / 1e9:.1f} TFLOP/s")
    del a, b, c
    return ms, flops


def fill_decode_state(torch, model, st, B, ctx):
    """Every KV cache slot and linear state of B sequences pre-filled as if
    `ctx` positions had been processed: K, V ~ N(0, 1); S ~ N(0, 1), z = |N(0, 1)|."""
    import synth
    from synth import device as sd
    from looped_weight_shared_loop_amd import _abi as A
    cfg = model.cfg
    Hkv, d = cfg.n_kv_heads, cfg.head_dim
    S_max = (st.max_seq + 63) // 64 * 64
    stream = torch.cuda.current_stream().cuda_stream
    sched = model.schedule()
    n_full = sum(1 for e in sched if e[2] == 1)
    n_lin = len(sched) - n_full
    for slot in range(n_full):      # K [B][Hkv][S_max][d], V^T [B][Hkv][d][S_max], positions < ctx
        kp, _ = st.region(A.REGION_K, slot)
        vp, _ = st.region(A.REGION_VT, slot)
        sd.fill_normal4(kp, True, (B, Hkv, ctx, d), (Hkv * S_max * d, S_max * d, d, 1), 2, synth.tid_kv(slot, "k"),
                        1.0, stream=stream)
        sd.fill_normal4(vp, True, (B, Hkv, ctx, d), (Hkv * d * S_max, d * S_max, 1, S_max), 2,
                        synth.tid_kv(slot, "v"), 1.0, stream=stream)
    for slot in range(n_lin):
        sp, _ = st.region(A.REGION_S, slot)
        zp, _ = st.region(A.REGION_Z, slot)
        sd.fill_normal4(sp, False, (1, 1, 1, B * Hkv * d * d), (0, 0, 0, 1), 2, synth.tid_linstate(slot, "S"), 1.0,
                        stream=stream)
        sd.fill_normal4(zp, False, (1, 1, 1, B * Hkv * d), (0, 0, 0, 1), 2, synth.tid_linstate(slot, "z"), 1.0,
                        absval=True, stream=stream)
    st.set_length(ctx)


def time_decode_pipelined(L, torch, model, B, ctx, calls, warmup):
    """Pass-pipelined decode: n_passes cohorts of B sequences, each call runs
    the looped block once for all cohorts' rows and returns one cohort's
    logits (B tokens per call in steady state)."""
    import synth
    from synth import device as sd
    G = model.cfg.n_passes
    st = model.new_state(G * B, ctx + warmup + calls + 2)
    fill_decode_state(torch, model, st, G * B, ctx)
    toks = torch.empty(warmup + calls + G, B, dtype=torch.int32, device="cuda")
    sd.fill_tensor_uniform_int(toks, 1, synth.TID_TOKENS + 300, model.cfg.vocab)
    model.workspace(G * B, G * B, st.max_seq)
    out = torch.empty(B, model.cfg.vocab, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for i in range(G - 1 + warmup):           # fill the pipeline, then warm up
        model.decode_pipelined(st, toks[i], out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    left = []
    e0.record()
    for i in range(calls):
        left.append(model.decode_pipelined(st, toks[G - 1 + warmup + i], out)[1])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    assert all(x >= 0 for x in left)          # every timed call returned a cohort's logits
    st.check()
    assert torch.isfinite(out).all().item()
    log(f"pipelined decode {G} x B={B} ctx={ctx}: {ms:.2f} ms/call")
    st.close()
    return ms


def ragged_lengths(B, ctx):
    """Per-sequence lengths of the ragged decode batch: spread over
    [ctx / 2, ctx] by a fixed stride permutation (every length distinct)."""
    half = ctx // 2
    return [half + (b * 7919) % (half + 1) for b in range(B)]


def time_decode(L, torch, model, B, ctx, steps, warmup, lengths=None):
    import synth
    from synth import device as sd
    st = model.new_state(B, ctx + warmup + steps + 1)
    cfg = model.cfg
    fill_decode_state(torch, model, st, B, ctx)
    if lengths is not None:              # ragged: sequence b holds lengths[b] <= ctx positions
        for b, n in enumerate(lengths):
            st.set_seq_length(b, n)
    toks = torch.empty(warmup + steps, B, dtype=torch.int32, device="cuda")
    sd.fill_tensor_uniform_int(toks, 1, synth.TID_TOKENS + 100, cfg.vocab)
    model.workspace(B, B, st.max_seq)
    torch.cuda.synchronize()
    for i in range(warmup):
        model.decode_step(st, toks[i])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        out = model.decode_step(st, toks[warmup + i])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    st.check()
    assert torch.isfinite(out).all().item()
    log(f"decode B={B} ctx={ctx}{' ragged' if lengths else ''}: {ms:.2f} ms/step")
    st.close()
    return ms


# one 9B-width group [linear x3, full] looped twice (8 executions); no embed or head
GROUP = dict(NINE_B, vocab=1024, n_layers=4, loop_start=0, loop_end=4)
MHC_BYTES_PER_TOKEN = 49184    # read X (2C), y (C); write X' (2C), u (C): bf16, C = 4096; + maps


def time_mhc_isolated(torch, T=65536, iters=10):
    """The mHC site kernel alone (mid-loop form) over T tokens of two 4096-wide
    bf16 streams: read X and the sublayer output y, write X' = H_res X +
    H_post y and u = RMSNorm(H_pre' X'), with the next site's maps from the
    projection and 20 Sinkhorn iterations.  The incoming maps are synthetic
    values in [0, 1) (they do not change the traffic)."""
    import synth
    from synth import device as sd
    from looped_weight_shared_loop_amd import _abi as A
    C = NINE_B["hidden"]
    X = torch.empty(T, 2, C, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    u = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(8, 2 * C, dtype=torch.float32, device="cuda")
    b = torch.empty(8, dtype=torch.float32, device="cuda")
    sd.fill_tensor_normal(X, 4, 1, 1.0)
    sd.fill_tensor_normal(y, 4, 2, 1.0)
    sd.fill_tensor_normal(w, 4, 3, 0.02)
    sd.fill_tensor_normal(b, 4, 4, 0.02)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    maps_in = torch.rand(T, 8, device="cuda", generator=gen)
    maps_out = torch.empty(T, 8, dtype=torch.float32, device="cuda")
    gamma = torch.ones(C, dtype=torch.float32, device="cuda")
    nb = A.loop_op_mhc_bytes(C)
    scr = torch.empty(nb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    f = lambda: A.loop_op_mhc(A.LOOP_BF16, A.LOOP_MHC_MID, T, C, 20, 1e-6, y.data_ptr(), None, X.data_ptr(),
                              maps_in.data_ptr(), maps_out.data_ptr(), w.data_ptr(), b.data_ptr(), gamma.data_ptr(),
                              u.data_ptr(), scr.data_ptr(), nb, stream)
    for _ in range(2):
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        f()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    assert torch.isfinite(maps_out).all().item()
    log(f"mHC isolated T={T}: {ms:.3f} ms")
    del X, y, u
    return ms


def time_group(L, torch, S=8192, iters=3):
    """One 9B-width group [lin, lin, lin, full] looped twice under two-stream
    mHC (8 executions), B=1, S=8192, inputs h ~ N(0, 1) passed as embeddings,
    final hidden states returned (no embedding lookup, no head)."""
    import synth
    from synth import device as sd
    cfg = L.ModelConfig(**GROUP)
    model = L.LoopModel(cfg, L.random_weights(cfg, 0))
    st = model.new_state(1, S)
    emb = torch.empty(1, S, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    sd.fill_tensor_normal(emb, 1, synth.TID_EMBEDS_IN, 1.0)
    model.workspace(1, S, S)
    out = model.prefill(st, embeds=emb, hidden_out=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        out = model.prefill(st, embeds=emb, hidden_out=True)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    st.check()
    assert torch.isfinite(out).all().item()
    log(f"group x2 S={S}: {ms:.2f} ms")
    st.close()
    model.close()
    return ms


TINY = dict(vocab=512, hidden=256, ffn=768, n_heads=4, n_kv_heads=4, head_dim=64, n_layers=8, loop_start=2,
            loop_end=6, n_passes=2, dtype="fp32")


def time_d256(L, torch, args):
    """The 9B shape with the page's head layout (16 query / 4 KV heads of 256):
    prefill at the bench length and the B=32 decode step."""
    cfg = L.ModelConfig(**NINE_B_D256)
    log("generating random-init 9B-shape weights, 16 x 256 heads")
    model = L.LoopModel(cfg, L.random_weights(cfg, 0))
    torch.cuda.synchronize()
    S = args.seq
    ms = time_prefill(L, torch, model, S, 2, 1)
    flops, _, attn_f, _ = prefill_flops(NINE_B_D256, S)
    out = {"heads": "16 q / 4 kv x 256", "prefill_ms": round(ms, 3), "prefill_tokens_per_s": round(S / (ms / 1e3), 1),
           "prefill_tflops": round(flops / (ms / 1e3) / 1e12, 1),
           "prefill_mfma_frac": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if not args.no_decode:
        dms = time_decode(L, torch, model, args.decode_batch, args.decode_ctx, args.decode_steps, 3)
        tot, _, _, _ = decode_bytes(NINE_B_D256, args.decode_batch, args.decode_ctx)
        gbs = tot / (dms / 1e3) / 1e9
        out.update({"decode_ms_per_step": round(dms, 3), "decode_tokens_per_s": round(args.decode_batch / (dms / 1e3), 1),
                    "decode_algorithmic_gb_per_step": round(tot / 1e9, 2), "decode_hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
    del model
    torch.cuda.empty_cache()
    return out


def time_tiny(L, torch, S=128, iters=20):
    """The tiny looped decoder (8 stored layers, block [2, 6) twice: 12
    executions; fp32): latency of one B=1 prefill of S=128 tokens (last-row
    logits) and of one decode step after it."""
    import synth
    from synth import device as sd
    cfg = L.ModelConfig(**TINY)
    model = L.LoopModel(cfg, L.random_weights(cfg, 0))
    st = model.new_state(1, S + iters + 8)
    toks = torch.empty(1, S + iters + 8, dtype=torch.int32, device="cuda")
    sd.fill_tensor_uniform_int(toks, 1, synth.TID_TOKENS, cfg.vocab)
    p = toks[:, :S].contiguous()
    for _ in range(3):
        model.prefill(st, p)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        model.prefill(st, p)
    e1.record()
    torch.cuda.synchronize()
    pre_ms = e0.elapsed_time(e1) / iters
    dec = [toks[:, S + i].contiguous() for i in range(iters + 2)]
    model.decode_step(st, dec[0])
    model.decode_step(st, dec[1])
    torch.cuda.synchronize()
    e0.record()
    for i in range(iters):
        model.decode_step(st, dec[2 + i])
    e1.record()
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / iters
    st.check()
    log(f"tiny: prefill S={S} {pre_ms:.3f} ms, decode step {dec_ms:.3f} ms")
    st.close()
    model.close()
    return pre_ms, dec_ms


def cpu_tiny_oracle(S=128):
    """The float64 oracle on the tiny configuration's full input (B=1, S=128)."""
    import oracle
    import synth
    cfg = oracle.tiny_config()
    W = oracle.make_weights(cfg, 0)
    toks = synth.uniform_int(1, synth.TID_TOKENS, (1, S), cfg.vocab)
    t0 = time.perf_counter()
    oracle.forward(cfg, W, toks)
    return time.perf_counter() - t0


def cpu_baseline(seq=128):
    """The oracle as it stands, on host cores, on a bounded sample: one 4-layer
    group [linear x3, full] at full 9B width looped twice (8 of the 56 layer
    executions) over `seq` tokens; scaled to a 56-execution tokens/s."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    cfg = oracle.group_config()
    W = oracle.make_weights(cfg, 0, cache_layers=4)
    for i in range(cfg.n_layers):
        W.layer(i)                          # generate outside the timed region
    emb = synth.normal_bf16_as_f32(1, synth.TID_EMBEDS_IN, (1, seq, cfg.hidden))
    t0 = time.perf_counter()
    oracle.forward(cfg, W, embeds=emb, hidden_out=True)
    dt = time.perf_counter() - t0
    per_token_56 = dt / seq * 56.0 / 8.0
    log(f"oracle sample: {dt:.1f} s for {seq} tokens x 8 executions")
    tiny_s = cpu_tiny_oracle()
    log(f"oracle, tiny config B=1 S=128: {tiny_s:.2f} s")
    return {"value": round(1.0 / per_token_56, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"float64 oracle, one 9B-width group [lin,lin,lin,full] looped twice (8 of 56 executions), "
                      f"B=1 S={seq}, {dt:.1f} s; scaled by 8/56 to the 56-execution model (head excluded)",
            "tiny": {"config": "tiny looped decoder (12 executions, fp32), B=1 S=128, last-row logits",
                     "oracle_s": round(tiny_s, 3), "tokens_per_s": round(128 / tiny_s, 1)}}


PROFILE_MODES = ("dominant", "prefill", "decode", "mhc", "group", "long", "prefill_d256", "decode_d256",
                 "decode_pipelined", "decode_ragged")


def profile_run(L, torch, args):
    """One instance of one workload after a 1 GiB device copy whose counter
    readings scale the HBM counters (FETCH_SIZE, WRITE_SIZE) to bytes:
      dominant  3 launches of the gate/up GEMM at M = 32768
      prefill   one Loop-9B prefill, B=1, S=32,768 (after one untimed warm-up call)
      decode    one decode step, B=32 at 32,768 pre-filled positions (after 2 warm-up steps)
      mhc       the mHC site alone, 65,536 tokens, 3 launches
      group     one 9B-width group looped twice, S=8,192 (after one warm-up call)
      long      one chunked prefill of 262,144 positions (8 chunks of 32,768)
      prefill_d256, decode_d256   prefill / decode with 16 query / 4 KV heads of 256
      decode_pipelined  one pass-pipelined call, 2 cohorts x 32 sequences at 32,768 positions
                (after the pipeline fill and 2 warm-up calls)
      decode_ragged     one decode step of the ragged batch (B=32, lengths 16,384-32,483)
    Prints the step it is in before each one, so a profiled run shows progress."""
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")     # 1 GiB
    dst = torch.empty_like(src)
    dst.copy_(src)                                                   # reads 1 GiB, writes 1 GiB
    torch.cuda.synchronize()
    del src, dst
    mode = args.profile
    log(f"profile {mode}: copy done")
    if mode == "dominant":
        time_dominant_gemm(L, torch, args.seq, iters=3)
    elif mode == "mhc":
        time_mhc_isolated(torch, iters=3)
    elif mode == "group":
        time_group(L, torch, iters=1)
    else:
        cfg = L.ModelConfig(**(NINE_B_D256 if mode.endswith("_d256") else NINE_B))
        model = L.LoopModel(cfg, L.random_weights(cfg, 0))
        torch.cuda.synchronize()
        log(f"profile {mode}: weights ready")
        if mode in ("prefill", "prefill_d256"):
            time_prefill(L, torch, model, args.seq, 1, 1)
        elif mode in ("decode", "decode_d256"):
            time_decode(L, torch, model, args.decode_batch, args.decode_ctx, 1, 2)
        elif mode == "decode_pipelined":
            time_decode_pipelined(L, torch, model, args.decode_batch, args.decode_ctx, 1, 2)
        elif mode == "decode_ragged":
            time_decode(L, torch, model, args.decode_batch, args.decode_ctx, 1, 2,
                        lengths=ragged_lengths(args.decode_batch, args.decode_ctx))
        elif mode == "long":
            time_long_prefill(L, torch, model, args.long_seq, args.long_chunk)
    torch.cuda.synchronize()
    print(json.dumps({"profile": mode, "done": True, "copy_bytes": 1 << 30}), flush=True)


# ------------------------------------------------------------------ rocprofv3 summaries
def _prof_rows(d, suffix):
    """Rows of the rocprofv3 CSV under directory d whose name ends in suffix,
    in dispatch order."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _kname(n):
    n = n.split("(")[0] if not n.startswith("(") else n.split(")::", 1)[-1].split("(")[0]
    return n.replace("void ", "").strip()


_ATTN_OR_LIN = ("attn_prefill_dma", "attn_prefill_d256", "attn_decode_mfma", "attn_combine", "lin_out_bf", "lin_decode_kernel",
                "lin_output", "attn_f32", "kv_append")


def _labels(names):
    """Names the projection of each GEMM launch from the driver's launch order:
    a plain-store GEMM after a norm or mHC kernel is the QKV projection of a
    linear-attention layer, after attention it is the O projection, after the
    gate/up GEMM (or its split-K reduction) it is the down projection."""
    out, prev = [], ""
    for n in names:
        lab = n
        if any(k in n for k in ("gemm_w16_kernel<", "gemm_skinny_rs_kernel<", "gemm_dma_kernel<")):
            epi = n.split("<")[1].split(",")[0].split(">")[0]
            kind = "skinny, weights streamed once" if "skinny" in n else "256-row tiles"
            if epi == "3":
                lab = f"gemm gate/up + SwiGLU ({kind}) {n}"
            elif epi == "2":
                lab = f"gemm QKV, full-attention layers ({kind}) {n}"
            elif epi == "1":
                lab = f"gemm head ({kind}) {n}"
            elif any(k in prev for k in _ATTN_OR_LIN):
                lab = f"gemm o ({kind}) {n}"
            elif "<3" in prev and "gemm" in prev:
                lab = f"gemm down ({kind}) {n}"
            else:
                lab = f"gemm QKV, linear-attention layers ({kind}) {n}"
        out.append(lab)
        if not n.startswith("at::") and "rocclr" not in n:
            prev = n
    return out


def _scope(names, scope, marker):
    """Index range summarized: everything after the 1 GiB reference copy
    ('all'), from the last launch of the marker kernel on ('last'), or from
    its launch N + 1 on ('after:N', e.g. past N untimed warm-up launches)."""
    first = next(i for i, n in enumerate(names) if n == "__amd_rocclr_copyBuffer") + 1
    if scope == "all":
        return first, len(names)
    idx = [i for i, n in enumerate(names) if marker in n and i >= first]
    if scope.startswith("after:"):
        k = int(scope.split(":")[1])
        return (idx[k] if k < len(idx) else len(names)), len(names)
    return (idx[-1] if idx else first), len(names)


def summarize(kind, dirs, scope, marker, title):
    import collections
    lines = [f"# {title}"]
    if kind == "trace":
        rows = _prof_rows(dirs[0], "kernel_trace.csv")
        names = [_kname(r["Kernel_Name"]) for r in rows]
        a, b = _scope(names, scope, marker)
        labs = _labels(names)
        agg = collections.OrderedDict()
        for i in range(a, b):
            if names[i].startswith("at::") or "rocclr" in names[i]:
                continue
            dt = (int(rows[i]["End_Timestamp"]) - int(rows[i]["Start_Timestamp"])) / 1e6
            e = agg.setdefault(labs[i], [0, 0.0])
            e[0] += 1
            e[1] += dt
        tot = sum(v[1] for v in agg.values())
        span = (int(rows[b - 1]["End_Timestamp"]) - int(rows[a]["Start_Timestamp"])) / 1e6
        lines.append(f"# library kernels: {tot:.3f} ms of kernel time; first start to last end {span:.3f} ms")
        lines.append("# kernel (projection named from the launch order) | launches | average ms | total ms | share")
        for k, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
            lines.append(f"{k[:96]:96s} | {c:5d} | {t / c:9.4f} | {t:9.3f} | {100 * t / tot:5.1f}%")
    elif kind == "mfma":
        rows = _prof_rows(dirs[0], "counter_collection.csv")
        per = collections.OrderedDict()
        for r in rows:
            e = per.setdefault(int(r["Dispatch_Id"]), {"name": _kname(r["Kernel_Name"]),
                                                        "t": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))})
            e[r["Counter_Name"]] = float(r["Counter_Value"])
        disp = list(per.values())
        names = [e["name"] for e in disp]
        a, b = _scope(names, scope, marker)
        labs = _labels(names)
        agg = collections.OrderedDict()
        for i in range(a, b):
            e = disp[i]
            if e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) == 0:
                continue
            g = agg.setdefault(labs[i], collections.defaultdict(float))
            g["n"] += 1
            for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
                      "GRBM_GUI_ACTIVE"):
                g[c] += e.get(c, 0.0)
            g["t"] += e["t"]
        lines.append("# MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCC x 1024 SIMDs); VALUBusy ="
                     " SQ_ACTIVE_INST_VALU / 256 CUs / GRBM_GUI_ACTIVE per XCC (rocprofv3's derived metrics);"
                     " GRBM_GUI_ACTIVE is the sum over the 8 XCCs")
        lines.append("# clock = GUI-active cycles per XCC / kernel duration under counter collection")
        lines.append("# kernel | launches | bf16 MFMA FLOP per launch (MOPS_BF16 x 512) | MfmaUtil | VALUBusy | clock GHz")
        tot_f = 0.0
        for k, g in sorted(agg.items(), key=lambda kv: -kv[1]["SQ_INSTS_VALU_MFMA_MOPS_BF16"]):
            n, gui = g["n"], g["GRBM_GUI_ACTIVE"] / 8
            tot_f += g["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            lines.append(f"{k[:96]:96s} | {int(n):5d} | {g['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / n:10.4e} | "
                         f"{g['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * 1024):6.3f} | "
                         f"{g['SQ_ACTIVE_INST_VALU'] / 256 / gui:6.3f} | {gui / g['t']:5.2f}")
        lines.append(f"# bf16 MFMA FLOP counted in the scope: {tot_f:.4e}")
    elif kind == "hbm":
        f = _prof_rows(dirs[0], "counter_collection.csv")
        w = _prof_rows(dirs[1], "counter_collection.csv")
        f = [(_kname(r["Kernel_Name"]), float(r["Counter_Value"])) for r in f if r["Counter_Name"] == "FETCH_SIZE"]
        w = [(_kname(r["Kernel_Name"]), float(r["Counter_Value"])) for r in w if r["Counter_Name"] == "WRITE_SIZE"]
        names = [n for n, _ in f]
        assert names == [n for n, _ in w], "the two runs launched different kernels"
        cf = next(v for n, v in f if n == "__amd_rocclr_copyBuffer")
        cw = next(v for n, v in w if n == "__amd_rocclr_copyBuffer")
        sf, sw = (1 << 30) / (cf * 1024), (1 << 30) / (cw * 1024)
        lines.append(f"# reference: a plain 1 GiB device copy reads FETCH_SIZE {cf:.1f} KiB (scale {sf:.4f}) and "
                     f"WRITE_SIZE {cw:.1f} KiB (scale {sw:.4f})")
        a, b = _scope(names, scope, marker)
        labs = _labels(names)
        agg = collections.OrderedDict()
        for i in range(a, b):
            if names[i].startswith("at::") or "rocclr" in names[i]:
                continue
            e = agg.setdefault(labs[i], [0, 0.0, 0.0])
            e[0] += 1
            e[1] += f[i][1] * 1024 * sf
            e[2] += w[i][1] * 1024 * sw
        tf = sum(v[1] for v in agg.values())
        tw = sum(v[2] for v in agg.values())
        lines.append(f"# library kernels in the scope: fetched {tf / 1e9:.3f} GB, written {tw / 1e9:.3f} GB, "
                     f"total {(tf + tw) / 1e9:.3f} GB")
        lines.append("# kernel | launches | fetched GB | written GB | GB per launch")
        for k, (c, x, y) in sorted(agg.items(), key=lambda kv: -(kv[1][1] + kv[1][2])):
            lines.append(f"{k[:96]:96s} | {c:5d} | {x / 1e9:9.3f} | {y / 1e9:8.3f} | {(x + y) / c / 1e9:8.4f}")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--seq", type=int, default=32768)
    ap.add_argument("--decode-batch", type=int, default=32)
    ap.add_argument("--decode-ctx", type=int, default=32768)
    ap.add_argument("--decode-steps", type=int, default=16)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-pipelined", action="store_true", help="skip the pass-pipelined decode")
    ap.add_argument("--long-seq", type=int, default=262144,
                    help="one chunked prefill of this many positions (0: skip)")
    ap.add_argument("--long-chunk", type=int, default=32768)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-parts", action="store_true",
                    help="skip the mHC-isolated and one-group measurements")
    ap.add_argument("--cpu-seq", type=int, default=1536)
    ap.add_argument("--no-d256", action="store_true", help="skip the 16 x 256 head layout")
    ap.add_argument("--profile-dominant", action="store_true",
                    help="only a 1 GiB device copy (counter scale reference) and 3 launches of the dominant kernel")
    ap.add_argument("--profile", choices=PROFILE_MODES, default=None,
                    help="only a 1 GiB device copy (counter scale reference) and ONE run of this workload, "
                         "for rocprofv3 kernel traces and counters per configuration")
    ap.add_argument("--summarize", nargs="+", metavar=("KIND", "DIR"),
                    help="print a summary of rocprofv3 CSV output instead of running: trace DIR | mfma DIR | "
                         "hbm FETCH_DIR WRITE_DIR (no GPU needed)")
    ap.add_argument("--scope", default="last",
                    help="with --summarize: last (from the last --marker launch), all (everything after the "
                         "reference copy) or after:N (from --marker launch N + 1 on)")
    ap.add_argument("--marker", default="embed_kernel", help="with --summarize: the kernel that starts a run")
    ap.add_argument("--title", default="rocprofv3 summary")
    args = ap.parse_args()
    if args.summarize:
        print(summarize(args.summarize[0], args.summarize[1:], args.scope, args.marker, args.title))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the looped-decoder path runs on one GPU (it has no cross-GPU path); run with --gpus 1", flush=True)
        sys.exit(2)

    import torch
    import looped_weight_shared_loop_amd as L

    if args.profile_dominant:
        args.profile = "dominant"
    if args.profile:
        profile_run(L, torch, args)
        return

    cfg = L.ModelConfig(**NINE_B)
    log("generating random-init 9B-shape weights on the device")
    model = L.LoopModel(cfg, L.random_weights(cfg, 0))
    torch.cuda.synchronize()

    S = args.seq
    ms = time_prefill(L, torch, model, S, args.steps, args.warmup)
    flops, gemm_f, attn_f, lin_f = prefill_flops(NINE_B, S)
    tok_s = S / (ms / 1e3)
    tflops = flops / (ms / 1e3) / 1e12

    g_ms, g_flops = time_dominant_gemm(L, torch, S)
    g_tflops = g_flops / (g_ms / 1e3) / 1e12
    traffic = dominant_traffic()

    result = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"Loop-9B-shape looped prefill (56 layer executions, 14 full-attention), "
                               f"B=1, S={S}, last-position logits", "batch": 1, "seq_len": S},
        "prefill": {"tflops": round(tflops, 1), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                    "algorithmic_tflop": round(flops / 1e12, 2), "gemm_tflop": round(gemm_f / 1e12, 2),
                    "attention_tflop": round(attn_f / 1e12, 2), "linear_tflop": round(lin_f / 1e12, 3)},
        "roofline": {"kernel": "gemm_w16_kernel<EPI_SWIGLU> (gate/up, M=%d N=24576 K=4096)" % S, "bound": "mfma",
                     "achieved": round(g_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": (None if S != 32768 or traffic is None else round(traffic)),
                     "algorithmic_bytes": (S * 4096 + 24576 * 4096 + S * 12288) * 2,
                     "avg_launch_ms": round(g_ms, 4)},
    }
    if not args.no_decode:
        dms = time_decode(L, torch, model, args.decode_batch, args.decode_ctx, args.decode_steps, 3)
        tot, w, kv, lin = decode_bytes(NINE_B, args.decode_batch, args.decode_ctx)
        gbs = tot / (dms / 1e3) / 1e9
        result["decode"] = {"tokens_per_s": round(args.decode_batch / (dms / 1e3), 1), "ms_per_step": round(dms, 3),
                            "batch": args.decode_batch, "context": args.decode_ctx,
                            "algorithmic_gb_per_step": round(tot / 1e9, 2), "achieved_gbs": round(gbs, 1),
                            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    if not args.no_decode:
        lens = ragged_lengths(args.decode_batch, args.decode_ctx)
        rms = time_decode(L, torch, model, args.decode_batch, args.decode_ctx, args.decode_steps, 3, lens)
        _, w, _, lin = decode_bytes(NINE_B, args.decode_batch, args.decode_ctx)
        _, _, kv1, _ = decode_bytes(NINE_B, 1, 1)             # K and V bytes of one position, all full slots
        rtot = w + lin + kv1 * sum(lens)
        rgbs = rtot / (rms / 1e3) / 1e9
        result["decode_ragged"] = {"tokens_per_s": round(args.decode_batch / (rms / 1e3), 1),
                                   "ms_per_step": round(rms, 3), "batch": args.decode_batch,
                                   "lengths": f"{min(lens)}..{max(lens)}, mean {sum(lens) / len(lens):.0f}",
                                   "algorithmic_gb_per_step": round(rtot / 1e9, 2), "achieved_gbs": round(rgbs, 1),
                                   "hbm_frac": round(rgbs / PEAK_HBM_GBS, 4)}
    if not args.no_decode and not args.no_pipelined:
        pms = time_decode_pipelined(L, torch, model, args.decode_batch, args.decode_ctx, args.decode_steps, 2)
        ptot, pw, _, _ = decode_pipelined_bytes(NINE_B, args.decode_batch, args.decode_ctx)
        pgbs = ptot / (pms / 1e3) / 1e9
        result["decode_pipelined"] = {
            "cohorts": NINE_B["n_passes"], "cohort_batch": args.decode_batch, "context": args.decode_ctx,
            "ms_per_call": round(pms, 3), "tokens_per_s": round(args.decode_batch / (pms / 1e3), 1),
            "algorithmic_gb_per_call": round(ptot / 1e9, 2), "weight_gb_per_call": round(pw / 1e9, 2),
            "achieved_gbs": round(pgbs, 1), "hbm_frac": round(pgbs / PEAK_HBM_GBS, 4)}
    if args.long_seq > 0:
        lms = time_long_prefill(L, torch, model, args.long_seq, args.long_chunk)
        lf, lg, la, ll = prefill_flops(NINE_B, args.long_seq)
        result["prefill_long"] = {"seq_len": args.long_seq, "chunk": args.long_chunk, "ms": round(lms, 1),
                                  "tokens_per_s": round(args.long_seq / (lms / 1e3), 1),
                                  "tflops": round(lf / (lms / 1e3) / 1e12, 1),
                                  "mfma_frac": round(lf / (lms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                  "algorithmic_tflop": round(lf / 1e12, 1), "attention_tflop": round(la / 1e12, 1)}
    if not args.no_parts:
        mms = time_mhc_isolated(torch)
        mgb = 65536 * MHC_BYTES_PER_TOKEN / (mms / 1e3) / 1e9
        result["mhc_isolated"] = {"tokens": 65536, "ms": round(mms, 4), "algorithmic_gb": round(65536 * MHC_BYTES_PER_TOKEN / 1e9, 3),
                                  "achieved_gbs": round(mgb, 1), "hbm_frac": round(mgb / PEAK_HBM_GBS, 4)}
        del model
        torch.cuda.empty_cache()
        gms = time_group(L, torch)
        _, gg, ga, gl = prefill_flops(GROUP, 8192)
        gf = gg + ga + gl
        result["group_x2"] = {"seq_len": 8192, "ms": round(gms, 3), "tokens_per_s": round(8192 / (gms / 1e3), 1),
                              "algorithmic_tflop": round(gf / 1e12, 2),
                              "tflops": round(gf / (gms / 1e3) / 1e12, 1),
                              "mfma_frac": round(gf / (gms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if not args.no_d256:
        if "model" in locals():
            del model
        torch.cuda.empty_cache()
        result["heads_16x256"] = time_d256(L, torch, args)
    if not args.no_parts:
        tp, td = time_tiny(L, torch)
        result["tiny"] = {"config": "tiny looped decoder (8 stored layers, block [2,6) x2 = 12 executions, fp32), "
                                    "B=1", "prefill_s128_ms": round(tp, 4), "decode_step_ms": round(td, 4),
                          "prefill_tokens_per_s": round(128 / (tp / 1e3), 1)}
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seq)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
