"""Paged per-pass KV caches (every full-attention (layer, pass) slot a pool of
64-position pages, one block table per sequence for all slots).  A paged
state must give the same logits as a contiguous one, bit for bit: the same
values land in the caches and attention reads them in the same order.  Pages
are handed out shuffled and interleaved between sequences, only as many as
the positions need, with the unused table entries set to garbage (they are
clamped, and never read for a position that exists).  Serving shared-weight
loops is the gap one page names ("SenseTime Open-Sources Loop-9B: Same
Layers, Run Twice", closing paragraphs on costs)."""
import numpy as np
import pytest

import oracle
from gpu_common import build_pair, mini_bf16_config, need_gpu, rel, to_dev_tokens, tokens, torch

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def assign_pages(state, lengths, seed):
    """Gives each sequence's blocks [0, ceil(len / 64)) distinct pages in a
    shuffled order; every other table entry gets a garbage value."""
    rng = np.random.default_rng(seed)
    B, blocks = state.block_table.shape
    need = [(n + 63) // 64 for n in lengths]
    assert sum(need) <= state.n_pages
    perm = rng.permutation(state.n_pages)
    table = np.full((B, blocks), -7, np.int64)
    table[:, ::3] = 10 ** 6
    k = 0
    order = [(b, j) for j in range(max(need)) for b in range(B) if j < need[b]]   # interleaved
    for b, j in order:
        table[b, j] = perm[k]
        k += 1
    state.block_table.copy_(torch.from_numpy(table.astype(np.int32)))


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "bf16_d256"])
def test_paged_ragged_prefill_decode_matches_contiguous(dtype):
    """Ragged rows (prefill subsets, a continued chunk), then decode steps, on a
    paged and on a contiguous state: equal logits; the fp32 case also against
    the oracle.  Prefills of more than 64 rows store plain QKV rows and
    scatter K / V into the pages; shorter ones write the pages directly."""
    need_gpu()
    ocfg = {"fp32": lambda: oracle.tiny_config(n_kv_heads=2), "bf16": mini_bf16_config,
            "bf16_d256": lambda: mini_bf16_config(n_heads=4, n_kv_heads=1, head_dim=256)}[dtype]()
    model, Wo = build_pair(ocfg)
    lens, K = [70, 70, 133, 20], 3
    toks = tokens(4, max(lens) + K, ocfg.vocab, seed=81)
    max_seq = 200
    _say("paged vs contiguous", dtype, "lengths", lens)
    final = [n + K for n in lens]
    n_pages = sum((n + 63) // 64 for n in final) + 1
    sp = model.new_state(4, max_seq, n_pages=n_pages)
    assign_pages(sp, final, seed=3)
    sc = model.new_state(4, max_seq)
    outs = {}
    for name, st in (("paged", sp), ("contiguous", sc)):
        o = [model.prefill(st, to_dev_tokens(toks[:2, :70]), all_logits=True).cpu().numpy()]
        o.append(model.prefill(st, to_dev_tokens(toks[2:3, :64]), seq0=2, all_logits=True).cpu().numpy())
        o.append(model.prefill(st, to_dev_tokens(toks[2:3, 64:133]), seq0=2, cont=True, all_logits=True)
                 .cpu().numpy())
        o.append(model.prefill(st, to_dev_tokens(toks[3:4, :20]), seq0=3).cpu().numpy())
        for k in range(K):
            step = np.array([toks[b, lens[b] + k] for b in range(4)], np.int32)
            o.append(model.decode_step(st, to_dev_tokens(step)).cpu().numpy())
        st.check()
        outs[name] = o
    for a, b in zip(outs["paged"], outs["contiguous"]):
        assert np.array_equal(a, b)
    assert sp.lengths == sc.lengths == final
    if dtype == "fp32":
        for b in range(4):
            ref = oracle.forward(ocfg, Wo, toks[b:b + 1, :final[b]], all_logits=True)[0]
            for k in range(K):
                assert rel(outs["paged"][4 + k][b:b + 1], ref[lens[b] + k][None]) < 1e-5


def test_paged_pipelined_decode_matches_contiguous():
    """The pass-pipelined decode on a paged state (cohort K/V appended through
    the table) equals the contiguous state's calls bit for bit."""
    need_gpu()
    ocfg = mini_bf16_config()
    model, _ = build_pair(ocfg)
    G, Bc, S, calls = 2, 2, 40, 5
    toks = tokens(G * Bc, S + calls + 2, ocfg.vocab, seed=83)
    final = [S + calls] * (G * Bc)
    sp = model.new_state(G * Bc, 128, n_pages=sum((n + 63) // 64 for n in final) + 3)
    assign_pages(sp, final, seed=5)
    sc = model.new_state(G * Bc, 128)
    res = {}
    for name, st in (("paged", sp), ("contiguous", sc)):
        model.prefill(st, to_dev_tokens(toks[:, :S]))
        sent = [0] * G
        r = []
        for t in range(calls):
            e = t % G
            entered, left, out = model.decode_pipelined(st, to_dev_tokens(toks[e * Bc:(e + 1) * Bc, S + sent[e]]))
            sent[e] += 1
            r.append((entered, left, out.cpu().numpy().copy() if left >= 0 else None))
        res[name] = r
    for (e1, l1, o1), (e2, l2, o2) in zip(res["paged"], res["contiguous"]):
        assert (e1, l1) == (e2, l2)
        if o1 is not None:
            assert np.array_equal(o1, o2)


@pytest.mark.parametrize("S", [2900])
@pytest.mark.parametrize("heads", [(32, 8, 128), (16, 4, 256)], ids=["32x128", "16x256"])
def test_paged_9b_width_full_attention_prefill_and_decode(S, heads):
    """One looped full-attention layer at 9B width (32q / 8kv x 128 or 16q /
    4kv x 256) over 2,900 positions (46 pages per sequence, B=2): prefill
    through the QKV projection, the page scatter and the DMA-fed prefill
    attention, then decode steps through the decode attention, paged against
    contiguous, bit for bit; and the oracle."""
    need_gpu()
    ocfg = oracle.group_config(vocab=1024, n_layers=1, loop_start=0, loop_end=1, n_passes=1, attn_period=1,
                               n_heads=heads[0], n_kv_heads=heads[1], head_dim=heads[2])
    model, Wo = build_pair(ocfg, cache_layers=4)
    B, K = 2, 3
    toks = tokens(B, S + K, ocfg.vocab, seed=85)
    final = [S + K] * B
    sp = model.new_state(B, S + 64, n_pages=sum((n + 63) // 64 for n in final) + 2)
    assign_pages(sp, final, seed=7)
    sc = model.new_state(B, S + 64)
    outs = {}
    for name, st in (("paged", sp), ("contiguous", sc)):
        o = [model.prefill(st, to_dev_tokens(toks[:, :S])).cpu().numpy()]
        for k in range(K):
            o.append(model.decode_step(st, to_dev_tokens(toks[:, S + k])).cpu().numpy())
        outs[name] = o
    for a, b in zip(outs["paged"], outs["contiguous"]):
        assert np.array_equal(a, b)
    ref = oracle.forward(ocfg, Wo, toks[:1], all_logits=True)[0]     # sequence 0
    err = rel(outs["paged"][0][:1], ref[S - 1][None])
    _say("paged 9B-width prefill rel err", heads, err)
    assert err < 2e-2
    for k in range(K):
        assert rel(outs["paged"][1 + k][:1], ref[S + k][None]) < 2e-2


def test_paged_state_rules():
    L = need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    model, _ = build_pair(oracle.tiny_config())
    with pytest.raises(L.LoopError) as e:
        A.loop_state_bytes_paged(model.handle, 2, 64, 0)
    assert e.value.code == A.LOOP_ERR_INVALID_ARG
    nb = A.loop_state_bytes_paged(model.handle, 2, 64, 3)
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.LoopError) as e:
        A.loop_state_create_paged(model.handle, buf.data_ptr(), nb, 2, 64, 3, 0)
    assert e.value.code == A.LOOP_ERR_INVALID_ARG
    tbl = torch.zeros(2, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(L.LoopError) as e:
        A.loop_state_create_paged(model.handle, buf.data_ptr(), nb - 256, 2, 64, 3, tbl.data_ptr())
    assert e.value.code == A.LOOP_ERR_CAPACITY
    # one more page adds a K and a V^T page (64 positions x 4 KV heads x 64 x fp32) to each
    # of the 3 full-attention slots of the tiny schedule
    assert A.loop_state_bytes_paged(model.handle, 2, 64, 4) - nb == 3 * 2 * 64 * 4 * 64 * 4
