"""Host-side logic of bench.py, no GPU: the algorithmic FLOP and byte counts
the bench line divides by, and the rocprofv3 summarizer that writes the
tables under profiles/ (launch labelling, scopes, counter scaling), on
synthetic CSV files shaped like rocprofv3's."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

NINE_B = bench.NINE_B


def test_prefill_flops_by_hand():
    """56 executions of 4 projections, 14 causal full-attention executions,
    42 linear ones, and the head on one row (Loop-9B: layers 0-3, block
    4-27 twice, 28-31)."""
    S = 32768
    C, F, d, Hq, Hkv = 4096, 12288, 128, 32, 8
    params = (Hq + 2 * Hkv) * d * C + C * Hq * d + 2 * F * C + C * F
    assert params == 6144 * 4096 + 4096 * 4096 + 24576 * 4096 + 4096 * 12288
    tot, gemm, attn, lin = bench.prefill_flops(NINE_B, S)
    assert gemm == 2.0 * params * S * 56
    assert attn == 14 * 2.0 * S * S * d * Hq
    assert lin == 42 * S * (2.0 * d * d * Hkv + 2.0 * d * d * Hq + 2.0 * d * (Hq + Hkv))
    assert tot == gemm + attn + lin + 2.0 * 248320 * C
    # the page's 16 x 256 heads have the same projections and the same attention FLOPs
    t2, g2, a2, _ = bench.prefill_flops(bench.NINE_B_D256, S)
    assert g2 == gemm and a2 == attn


def test_decode_bytes_by_hand():
    tot, w, kv, lin = bench.decode_bytes(NINE_B, 32, 32768)
    per_layer = (6144 * 4096 + 4096 * 4096 + 24576 * 4096 + 4096 * 12288) * 2
    assert w == per_layer * 56 + 248320 * 4096 * 2
    assert kv == 14 * 32 * 8 * 32768 * 128 * 2 * 2
    assert lin == 42 * 32 * 8 * (128 * 128 + 128) * 4 * 2
    assert round(tot / 1e9, 2) == 85.19
    # the pipelined call reads every stored layer once
    ptot, pw, pkv, plin = bench.decode_pipelined_bytes(NINE_B, 32, 32768)
    assert pw == per_layer * 32 + 248320 * 4096 * 2 and pkv == kv and plin == lin


def _write(path, rows, fields):
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=fields)
        wr.writeheader()
        wr.writerows(rows)


# one synthetic run: the reference copy, then a prefill-like launch sequence
SEQ = ["__amd_rocclr_copyBuffer",
       "void lk::embed_kernel<unsigned short>(lk::EmbArgs)",
       "void lk::add_rmsnorm_kernel<unsigned short, 4>(lk::NormArgs)",
       "void lk::gemm_w16_kernel<0>(lk::GemmArgs)",           # QKV of a linear layer
       "lk::lin_out_bf<4, 128>(lk::LinArgs)",
       "void lk::gemm_w16_kernel<0>(lk::GemmArgs)",           # o
       "void lk::add_rmsnorm_kernel<unsigned short, 4>(lk::NormArgs)",
       "void lk::gemm_w16_kernel<3>(lk::GemmArgs)",           # gate/up
       "void lk::gemm_w16_kernel<0>(lk::GemmArgs)",           # down
       "void lk::gemm_w16_kernel<2>(lk::GemmArgs)",           # QKV of a full layer
       "lk::attn_prefill_dma(lk::AttnArgs)",
       "void lk::gemm_w16_kernel<0>(lk::GemmArgs)",           # o
       "void lk::gemm_skinny_rs_kernel<1, 1, 4>(lk::GemmArgs)"]


def test_summarize_trace_labels_and_scope(tmp_path):
    rows = []
    t = 1000
    for i, n in enumerate(SEQ):
        dur = 1000 * (i + 1)
        rows.append({"Dispatch_Id": i + 1, "Kernel_Name": n, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 10
    # a second run of the last four launches after another marker
    _write(tmp_path / "p_kernel_trace.csv", rows, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
    out = bench.summarize("trace", [str(tmp_path)], "all", "embed_kernel", "t")
    lines = out.splitlines()
    body = {l.split("|")[0].strip(): l for l in lines if not l.startswith("#")}
    assert any(k.startswith("gemm QKV, linear-attention layers") for k in body)
    assert any(k.startswith("gemm gate/up + SwiGLU") for k in body)
    assert any(k.startswith("gemm down") for k in body)
    assert any(k.startswith("gemm QKV, full-attention layers") for k in body)
    assert any(k.startswith("gemm head (skinny") for k in body)
    o = [l for k, l in body.items() if k.startswith("gemm o ")]
    assert len(o) == 1 and int(o[0].split("|")[1]) == 2          # both o projections, after attention
    # kernel time excludes the reference copy: sum of durations of launches 2..13 in microseconds
    total = sum(1000 * (i + 1) for i in range(1, len(SEQ))) / 1e6
    assert f"{total:.3f} ms of kernel time" in lines[1]


def test_summarize_hbm_scales_by_the_copy(tmp_path):
    names = SEQ[:4]
    fr, wr = [], []
    for i, n in enumerate(names):
        fetch = 524288.0 if i == 0 else 1000.0 * i            # the copy reads 1 GiB as half the KiB
        write = 1048576.0 if i == 0 else 500.0 * i
        base = {"Dispatch_Id": i + 1, "Kernel_Name": n}
        fr.append(dict(base, Counter_Name="FETCH_SIZE", Counter_Value=fetch))
        wr.append(dict(base, Counter_Name="WRITE_SIZE", Counter_Value=write))
    (tmp_path / "f").mkdir()
    (tmp_path / "w").mkdir()
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(tmp_path / "f" / "p_counter_collection.csv", fr, fields)
    _write(tmp_path / "w" / "p_counter_collection.csv", wr, fields)
    out = bench.summarize("hbm", [str(tmp_path / "f"), str(tmp_path / "w")], "all", "embed_kernel", "t")
    assert "scale 2.0000" in out and "scale 1.0000" in out
    # fetched: (1000 + 2000 + 3000) KiB x 1024 x 2, written (500 + 1000 + 1500) KiB x 1024
    tf, tw = 6000 * 1024 * 2 / 1e9, 3000 * 1024 / 1e9
    assert f"fetched {tf:.3f} GB, written {tw:.3f} GB" in out


def test_gemm_source_hash_ignores_comments(tmp_path, monkeypatch):
    """The traffic figure is tied to the GEMM source, not to its comments."""
    h = bench.gemm_source_hash()
    assert len(h) == 16 and all(ch in "0123456789abcdef" for ch in h)
    assert (bench.dominant_traffic() is None) == (h != bench.DOMINANT_COUNTERS["source_sha256_16"])


def test_bench_refuses_several_gpus():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stdout
