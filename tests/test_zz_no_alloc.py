"""loop_decode_step_noalloc (the decode step on the library's own static
device workspace, for callers that cannot allocate) against loop_decode_step
on a caller workspace: two states prefilled alike, then two decode calls in a
row on each, the second over fewer sequences.  The two entry points run the
same kernels on the same inputs, so the logits must agree bit for bit; a step
whose workspace exceeds the static array is refused before any launch."""
import numpy as np
import pytest

import oracle
from gpu_common import build_pair, mini_bf16_config, need_gpu, to_dev_tokens, tokens, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("which", ["tiny_fp32", "mini_bf16", "9b_width_bf16"])
def test_noalloc_decode_matches_decode_step(which):
    L = need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    if which == "tiny_fp32":
        ocfg = oracle.tiny_config(n_kv_heads=2)
    elif which == "mini_bf16":
        ocfg = mini_bf16_config()
    else:   # decode-shaped GEMMs split K over workgroups and leave partials in the workspace
        ocfg = oracle.group_config(vocab=1024, n_layers=4, loop_start=3, loop_end=4, n_passes=1)
    model, _ = build_pair(ocfg, cache_layers=4)
    B, S = 4, 40
    toks = tokens(B, S + 2, ocfg.vocab, seed=71)
    print("noalloc decode", which, flush=True)
    sa, sb = model.new_state(B, 64), model.new_state(B, 64)
    for st in (sa, sb):
        model.prefill(st, to_dev_tokens(toks[:, :S]))
    need = A.loop_workspace_bytes(model.handle, B, B, 64)
    print("workspace bytes of the step:", need, "static:", A.LOOP_NOALLOC_WORKSPACE_BYTES, flush=True)
    assert need <= A.LOOP_NOALLOC_WORKSPACE_BYTES
    out = torch.full((B, ocfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    # call 1: all four sequences; call 2: the first two (a smaller input)
    for n, col in ((B, S), (2, S + 1)):
        t = to_dev_tokens(toks[:n, col])
        ref = model.decode_step(sa, t).clone()
        out.fill_(float("nan"))
        model.decode_step_noalloc(sb, t, out)
        torch.cuda.synchronize()
        got = out[:n]
        assert torch.isfinite(got).all().item()
        assert torch.equal(got, ref), float((got - ref).abs().max())
        assert torch.isnan(out[n:]).all().item()       # rows past the call's batch untouched
    assert sa.lengths == sb.lengths == [S + 2, S + 2, S + 1, S + 1]


def test_noalloc_refuses_a_step_beyond_the_static_workspace():
    L = need_gpu()
    from looped_weight_shared_loop_amd import _abi as A
    ocfg = mini_bf16_config()
    model, _ = build_pair(ocfg)
    B = 1024
    need = A.loop_workspace_bytes(model.handle, B, B, 64)
    assert need > A.LOOP_NOALLOC_WORKSPACE_BYTES
    st = model.new_state(B, 64)
    st.set_length(8)
    toks = to_dev_tokens(np.zeros(B, np.int32))
    out = torch.empty(B, ocfg.vocab, dtype=torch.float32, device="cuda")
    with pytest.raises(L.LoopError) as e:
        model.decode_step_noalloc(st, toks, out)
    assert e.value.code == A.LOOP_ERR_WORKSPACE
    assert "static" in str(e.value)
    assert st.lengths == [8] * B
