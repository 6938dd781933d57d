"""Writes the stored expected values of the bf16 end-to-end parity tests.

Calls only the CPU oracle (``oracle/``) and the seeded input draws (``synth``);
nothing here touches the GPU library.  Run from the repository root:

    python tests/golden/make_golden.py loop9b   # ~6 min, ~30 GB of host memory
    python tests/golden/make_golden.py group    # ~5 min

    python tests/golden/make_golden.py group256 # ~2 min

loop9b -> tests/golden/loop9b_logits.npz
    The full Loop-9B shape (32 stored layers, block [4, 28) run twice: 56
    layer executions; vocabulary 248,320; pages: "SenseTime's Loop-9B runs its
    own layers twice, and gets a deeper model for free", section "The trick";
    "How Does SenseNova-Loop Get More Depth Without More Parameters?", section
    "What is the looped decoder in SenseNova-Loop?").  Weights seed 0, token
    ids seed 1, B = 2 sequences of 130 tokens.  The oracle's forward over all
    130 positions gives the logits of a 128-position prefill (rows 64 and 127)
    and of the two decode steps after it (rows 128 and 129): decode of token T
    is row T of the forward over tokens 0..T.  Stored for two oracle runs on
    the same bf16-valued weights and token ids: ``rounded`` (bf16 at the
    storage points, as the GPU path stores) and ``unrounded`` (float64
    between the steps: the exact-arithmetic result).

group -> tests/golden/group9b_hidden.npz
    One [linear, linear, linear, full] group at 9B width looped twice (8
    executions) on inputs N(0, 1) (seed 1), S = 200, hidden states out; the
    rounded result as bf16 bit patterns (it is bf16-valued), the unrounded one
    as float32.  Also how far the rounded oracle moves when one input element
    is moved by one bf16 ulp, at eight sites spread over positions and
    channels (max-row and row-RMS relative change per site).

group256 -> tests/golden/group9b_d256_hidden.npz
    The same group with the attention heads as one page gives them, 16 query
    and 4 KV heads of 256 ("How Does SenseNova-Loop Get More Depth Without
    More Parameters?", section on the hybrid attention pattern; the projection
    sizes equal those of 32 / 8 heads of 128): rounded and unrounded results.
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle          # noqa: E402
import synth           # noqa: E402
from oracle import model as M   # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))

LOOP9B_B, LOOP9B_T, LOOP9B_PREFILL = 2, 130, 128
LOOP9B_ROWS = (64, 127, 128, 129)
GROUP_S = 200
SENS_SITES = ((5, 17), (23, 4000), (51, 1024), (80, 2047), (111, 3), (150, 3333), (177, 640), (199, 2900))


def row_rms_rel(g, r):
    g = np.asarray(g, np.float64).reshape(-1, np.shape(g)[-1])
    r = np.asarray(r, np.float64).reshape(-1, np.shape(r)[-1])
    return (np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1))


def row_max_rel(g, r):
    g = np.asarray(g, np.float64).reshape(-1, np.shape(g)[-1])
    r = np.asarray(r, np.float64).reshape(-1, np.shape(r)[-1])
    return np.abs(g - r).max(axis=1) / np.abs(r).max(axis=1)


def make_loop9b():
    cfg = oracle.nine_b_config()
    cfg_exact = oracle.nine_b_config(round_storage=False)
    W = M.make_weights(cfg, 0, lazy=True, cache_layers=cfg.n_layers)
    toks = synth.uniform_int(1, synth.TID_TOKENS, (LOOP9B_B, LOOP9B_T), cfg.vocab)
    rows = list(LOOP9B_ROWS)
    out = {}
    for name, c in (("rounded", cfg), ("unrounded", cfg_exact)):
        t0 = time.time()
        st = M.State()
        lg = M.forward(c, W, toks, state=st, all_logits=True)
        assert len(st.calls) == 2 * 56 and st.length == LOOP9B_T   # 56 executions, two sublayers each
        out[name] = lg[:, rows, :].astype(np.float32)
        print(f"{name}: {time.time() - t0:.0f} s", flush=True)
    err_max = row_max_rel(out["rounded"], out["unrounded"]).reshape(LOOP9B_B, len(rows))
    err_rms = row_rms_rel(out["rounded"], out["unrounded"]).reshape(LOOP9B_B, len(rows))
    meta = dict(config="Loop-9B shape, bf16, weights seed 0, token ids seed 1", B=LOOP9B_B, T=LOOP9B_T,
                prefill=LOOP9B_PREFILL, rows=rows,
                rounded_vs_unrounded_max_row=err_max.tolist(), rounded_vs_unrounded_row_rms=err_rms.tolist())
    print(json.dumps(meta, indent=1), flush=True)
    np.savez_compressed(os.path.join(HERE, "loop9b_logits.npz"), tokens=toks.astype(np.int32),
                        rows=np.array(rows, np.int32), rounded=out["rounded"], unrounded=out["unrounded"],
                        meta=np.array(json.dumps(meta)))


def make_group(heads=None):
    kw = dict(n_heads=heads[0], n_kv_heads=heads[1], head_dim=heads[2]) if heads else {}
    cfg = oracle.group_config(**kw)
    cfg_exact = oracle.group_config(round_storage=False, **kw)
    W = M.make_weights(cfg, 0, cache_layers=4)
    emb = synth.normal_bf16_as_f32(1, synth.TID_EMBEDS_IN, (1, GROUP_S, cfg.hidden))
    t0 = time.time()
    ref = M.forward(cfg, W, embeds=emb, hidden_out=True)
    exact = M.forward(cfg_exact, W, embeds=emb, hidden_out=True)
    print(f"group: {time.time() - t0:.0f} s", flush=True)
    assert np.array_equal(M.round_bf16(ref), ref)
    bits = synth.f32_to_bf16_bits(ref.astype(np.float32))
    if heads:
        meta = dict(config=f"one 9B-width group [lin, lin, lin, full] looped twice, {heads[0]} q / {heads[1]} kv "
                    f"heads of {heads[2]}, bf16, weights seed 0, inputs seed 1",
                    S=GROUP_S, heads=list(heads), rounded_vs_unrounded_max_row=float(row_max_rel(ref, exact).max()),
                    rounded_vs_unrounded_row_rms=float(row_rms_rel(ref, exact).mean()))
        print(json.dumps(meta, indent=1), flush=True)
        np.savez_compressed(os.path.join(HERE, f"group9b_d{heads[2]}_hidden.npz"), rounded_bf16_bits=bits,
                            unrounded=exact.astype(np.float32), meta=np.array(json.dumps(meta)))
        return
    sens = []
    for (t, c) in SENS_SITES:
        e2 = emb.copy()
        e2[0, t, c] = np.float32(M.round_bf16(e2[0, t, c] * (1 + 2 ** -7)))
        assert e2[0, t, c] != emb[0, t, c]
        p = M.forward(cfg, W, embeds=e2, hidden_out=True)
        assert np.array_equal(p[0, :t], ref[0, :t])          # causality: earlier rows untouched
        sens.append(dict(position=t, channel=c, max_row=float(row_max_rel(p, ref).max()),
                         row_rms=float(row_rms_rel(p[0, t:], ref[0, t:]).mean())))
        print(sens[-1], flush=True)
    meta = dict(config="one 9B-width group [lin, lin, lin, full] looped twice, bf16, weights seed 0, inputs seed 1",
                S=GROUP_S, rounded_vs_unrounded_max_row=float(row_max_rel(ref, exact).max()),
                rounded_vs_unrounded_row_rms=float(row_rms_rel(ref, exact).mean()), one_ulp_sensitivity=sens)
    print(json.dumps(meta, indent=1), flush=True)
    np.savez_compressed(os.path.join(HERE, "group9b_hidden.npz"), rounded_bf16_bits=bits,
                        unrounded=exact.astype(np.float32), meta=np.array(json.dumps(meta)))


if __name__ == "__main__":
    which = sys.argv[1:] or ["group", "loop9b"]
    for w in which:
        {"loop9b": make_loop9b, "group": make_group, "group256": lambda: make_group((16, 4, 256))}[w]()
