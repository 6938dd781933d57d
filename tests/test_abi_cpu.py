"""Host-side checks of the C ABI: the library loads, exports every entry point
include/loop.h declares, and rejects bad configurations before touching a
device.  No compute call is made (no GPU here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("loop.h", "loop_ops.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(loop_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("loop_model_create", "loop_prefill", "loop_decode_step", "loop_state_bytes",
              "loop_workspace_bytes", "loop_state_create", "loop_last_error", "loop_op_gemm", "loop_op_mhc",
              "loop_op_attention", "loop_op_attention_decode", "loop_op_linear"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from looped_weight_shared_loop_amd import _abi
    lib = ctypes.CDLL(_abi.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing
    assert set(_declared()) == set(_abi.SYMBOLS), "binding and header disagree"


def test_synth_library_exports():
    from synth import device
    lib = ctypes.CDLL(device.LIB_PATH)
    assert hasattr(lib, "synth_fill_normal4") and hasattr(lib, "synth_fill_uniform_int")


def _cfg(**kw):
    from looped_weight_shared_loop_amd import ModelConfig
    base = dict(vocab=512, hidden=256, ffn=768, n_heads=4, n_kv_heads=4, head_dim=64, n_layers=8,
                loop_start=2, loop_end=6, dtype="fp32")
    base.update(kw)
    return ModelConfig(**base)


def _create(cfg, n_layers=None):
    from looped_weight_shared_loop_amd import _abi as A
    layers = (A.loop_layer_weights * cfg.n_layers)()
    w = A.loop_weights(16, 16, 16, ctypes.cast(layers, ctypes.POINTER(A.loop_layer_weights)),
                       cfg.n_layers if n_layers is None else n_layers)
    return A.loop_model_create(cfg.to_c(), w)


@pytest.mark.parametrize("kw,code", [
    (dict(loop_start=5, loop_end=3), -1),
    (dict(loop_end=9), -1),
    (dict(n_passes=0), -1),
    (dict(attn_period=0), -1),
    (dict(rms_eps=0.0), -1),
    (dict(n_kv_heads=3), -2),
    (dict(n_heads=32, n_kv_heads=2), -2),
    (dict(hidden=260), -2),
    (dict(hidden=8192), -2),
    (dict(head_dim=96), -2),
    (dict(dtype="bf16"), -2),                 # bf16 needs head_dim 128 or 256
    (dict(dtype="bf16", head_dim=128, hidden=200), -2),
    (dict(dtype="bf16", head_dim=128, hidden=256, n_heads=6, n_kv_heads=2), -2),   # group of 3 heads
    (dict(dtype="bf16", head_dim=256, hidden=256, n_heads=8, n_kv_heads=1), -2),   # 8 heads of 256 per group
    (dict(head_dim=256), -2),                 # float32 needs head_dim 64 or 128
    # weight matrices the 256-row GEMM tiles cannot address with 32-bit offsets: refused at
    # creation, before any call could fail part-way through a forward
    (dict(dtype="bf16", head_dim=128, hidden=4096, n_heads=32, n_kv_heads=8, ffn=12288, vocab=1 << 20), -2),
    (dict(dtype="bf16", head_dim=128, hidden=4096, n_heads=32, n_kv_heads=8, ffn=1 << 18, vocab=1024), -2),
])
def test_create_rejects_bad_configs(kw, code):
    from looped_weight_shared_loop_amd import LoopError
    with pytest.raises(LoopError) as e:
        _create(_cfg(**kw))
    assert e.value.code == code


def test_create_layer_count_mismatch():
    from looped_weight_shared_loop_amd import LoopError
    with pytest.raises(LoopError) as e:
        _create(_cfg(), n_layers=7)
    assert e.value.code == -1


def test_create_without_device_reports_no_device():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    from looped_weight_shared_loop_amd import LoopError
    with pytest.raises(LoopError) as e:
        _create(_cfg())
    assert e.value.code == -6
    with pytest.raises(LoopError) as e:
        _create(_cfg(dtype="bf16", vocab=248320, hidden=4096, ffn=12288, n_heads=32, n_kv_heads=8,
                     head_dim=128, n_layers=32, loop_start=4, loop_end=28))
    assert e.value.code == -6


def test_status_strings_and_null_arguments():
    from looped_weight_shared_loop_amd import _abi as A
    lib = A.lib()
    for code in range(0, -10, -1):
        assert A.loop_status_string(code) not in ("", "unknown status")
    assert A.loop_status_string(-42) == "unknown status"
    assert lib.loop_model_create(None, None, None) == A.LOOP_ERR_INVALID_ARG
    assert "null" in A.loop_last_error()
    assert lib.loop_prefill(None, None, None, 0, None, None, 1, 1, 0, None, None) == A.LOOP_ERR_INVALID_ARG
    assert lib.loop_decode_step(None, None, None, 0, None, 1, None, None) == A.LOOP_ERR_INVALID_ARG
    assert lib.loop_state_bytes(None, 1, 1, None) == A.LOOP_ERR_INVALID_ARG


def test_op_level_validation_without_device():
    """Argument checks of the op-level entry points run before any launch."""
    from looped_weight_shared_loop_amd import _abi as A
    lib = A.lib()
    assert lib.loop_op_gemm(7, 0, 1, 1, 1, None, 1, None, 1, None, 1, 0, None, 0, None) == A.LOOP_ERR_INVALID_ARG
    assert lib.loop_op_gemm(1, 0, 64, 256, 64, None, 64, None, 64, None, 256, 0, None, 0, None) == A.LOOP_ERR_INVALID_ARG
    assert lib.loop_op_gemm(1, 3, 64, 256, 64, 16, 64, 16, 64, 16, 128, 100, None, 0, None) == A.LOOP_ERR_INVALID_ARG
    assert lib.loop_op_gemm(1, 0, 64, 256, 64, 24, 64, 16, 64, 16, 256, 0, None, 0, None) == A.LOOP_ERR_ALIGN
    assert lib.loop_op_gemm(1, 0, 8, 256, 256, 16, 256, 16, 256, 16, 256, 0, 24, 64, None) == A.LOOP_ERR_ALIGN
    # prefill-shaped bf16 (M > 64): output widths off the 256-column tile, and 256 fp32
    # output rows past 2^31 bytes (the tile's stores use 32-bit offsets), are shape errors
    assert lib.loop_op_gemm(1, 0, 128, 300, 128, 16, 128, 16, 128, 16, 300, 0, None, 0, None) == A.LOOP_ERR_SHAPE
    assert lib.loop_op_gemm(1, 1, 128, 256, 128, 16, 128, 16, 128, 16, 1 << 21, 0, None, 0, None) == A.LOOP_ERR_SHAPE
    # fp32 and prefill shapes need no split-K scratch
    assert lib.loop_op_gemm_bytes(0, 0, 8, 4096, 4096, 0) == 0
    assert lib.loop_op_gemm_bytes(1, 0, 64, 4096, 4096, 0) == 0
    assert lib.loop_op_mhc(1, 9, 1, 8, 20, 1e-6, None, None, 16, None, None, None, None, 16, 16, None, 0, None) == \
        A.LOOP_ERR_INVALID_ARG
    assert A.loop_op_mhc_bytes(4096) == 24 * 8192 * 2
    assert lib.loop_op_attention(1, 1, 10, 60, 64, 4, 2, 128, 16, 512, 16, 16, 16, 512, None) == \
        A.LOOP_ERR_INVALID_ARG      # pos0 + S beyond S_max
    assert lib.loop_op_linear(1, 1, 1, 8, 4, 3, 64, 1e-6, 16, 768, 16, 16, 0, 16, 256, 16, 1 << 20, None) == \
        A.LOOP_ERR_INVALID_ARG      # Hq % Hkv
    # at least one split per row, at most one per 64 cached keys (the device CU count sets the rest)
    nb = A.loop_op_attention_decode_bytes(32, 1, 32, 128, 32832)
    assert 32 * 32 * 130 * 4 <= nb <= 32 * 32 * (32832 // 64) * 130 * 4 and nb % (32 * 32 * 130 * 4) == 0
    assert A.loop_op_linear_bytes(1, 100, 8, 128) == 2 * 8 * (128 * 128 + 128) * 4
    # stream-K decode attention: bf16 only, starts present and inside S_max; the scratch holds at
    # least one partial slot per row plus the starts and the key prefix
    import numpy as np
    starts = np.array([100, 7000], np.int32)
    args = (2, 1, starts.ctypes.data, 8192, 32, 8, 128, 16, 6144, 16, 16, 16, 4096, 16, 1 << 24, None)
    assert lib.loop_op_attention_decode_stream_k(0, *args) == A.LOOP_ERR_INVALID_ARG          # float32
    assert lib.loop_op_attention_decode_stream_k(1, 2, 1, None, *args[3:]) == A.LOOP_ERR_INVALID_ARG
    bad = np.array([100, 9000], np.int32)                                                      # past S_max
    assert lib.loop_op_attention_decode_stream_k(1, 2, 1, bad.ctypes.data, *args[3:]) == A.LOOP_ERR_INVALID_ARG
    nbs = A.loop_op_attention_decode_stream_k_bytes(2, 1, 32, 8, 128)
    assert nbs >= 2 * 32 * 130 * 4 + 5 * 4
