"""Host-side logic of bench.py, on the CPU: the algorithmic byte and flop
counts against hand-counted values, the one-GPU guard, and the rule that a
committed traffic summary counts only while the kernel sources match it."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get_workload, small_workload  # noqa: E402


def test_algorithmic_counts_bf16():
    # Two sequences of 3 and 40 tokens, 2 heads, one query token, d_c 512:
    # a bf16 record is (512 + 64) * 2 = 1152 bytes.
    w = small_workload("deepseek_v3", batch=2, heads=2, seq_len=(3, 40), max_seq_len=64)
    a = bench.algorithmic(w, [3, 40])
    assert a["record_bytes"] == 1152
    assert a["tokens"] == 43
    assert a["cache_bytes"] == 43 * 1152
    # queries read by the decode: B * R * (d_c + d_r) * 2 with R = S_q * H = 2
    assert a["decode_bytes"] == 43 * 1152 + 2 * 2 * 576 * 2
    # scores (d_c + d_r) and values (d_c): 2 flops per multiply-add, every head, every visible token
    assert a["attn_flops"] == 2 * 2 * 43 * (2 * 512 + 64)


def test_algorithmic_counts_fp8_causal_tail():
    # e4m3 records carry one fp32 scale: 576 + 4 = 580 bytes.  With S_q = 4,
    # query s of a length-L sequence sees L - 4 + 1 + s tokens.
    w = small_workload("kimi_k2_fp8", batch=1, heads=1, seq_len=(10, 10), max_seq_len=64)
    a = bench.algorithmic(w, [10])
    assert a["record_bytes"] == 580
    assert a["cache_bytes"] == 10 * 580
    visible = sum(10 - 4 + 1 + s for s in range(4))  # 7 + 8 + 9 + 10
    assert a["attn_flops"] == 2 * 1 * visible * (2 * 512 + 64)


def test_headline_decode_bytes_match_the_roofline_unit():
    # 204545 visible tokens of the headline workload (seeded lengths) at 1152
    # bytes, plus 32 sequences' 128 query rows of 576 bf16 values.
    w = get_workload("deepseek_v3")
    from workloads.generate import make_inputs
    L = make_inputs(w, poison=False)["seq_lens"]
    a = bench.algorithmic(w, L)
    assert a["tokens"] == 204545
    assert a["decode_bytes"] == 204545 * 1152 + 32 * 128 * 576 * 2 == 240354432


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_traffic_counts_only_for_matching_sources(monkeypatch, tmp_path):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "decode_wide_kernel_wl_traffic.txt").write_text(
        "# header\nhbm_bytes_per_launch: 12345\nkernel_source_sha256: abc\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.measured_traffic("wl", "decode_wide_kernel") == 12345
    assert bench.measured_traffic("wl", "decode_f8_kernel") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "changed")
    assert bench.measured_traffic("wl", "decode_wide_kernel") is None
    assert bench.measured_traffic("missing", "decode_wide_kernel") is None


@pytest.mark.parametrize("name", bench.KERNEL_SOURCES)
def test_hashed_sources_exist(name):
    assert os.path.exists(os.path.join(ROOT, "head_latent_attention_absorbed_amd", "csrc", name))


def test_roofline_bound_follows_the_ridge():
    """The headline workload (about 242 flop/B) is reported against HBM, the
    4-token e4m3 workload (about 960 flop/B) against the MFMA peak of its
    products: e4m3 for the score product, bf16 for P . V."""
    from workloads.generate import make_inputs
    for name, bound in (("deepseek_v3", "hbm"), ("kimi_k2_fp8", "mfma")):
        w = get_workload(name)
        a = bench.algorithmic(w, make_inputs(w, poison=False)["seq_lens"])
        r = bench.roofline_of(a, 100.0, {"hbm_gbs": 6000.0, "mfma_bf16_tflops": 2000.0}, w)
        assert r["bound"] == bound, (name, r)
        us = 100e-6
        if bound == "hbm":
            assert r["achieved"] == round(a["decode_bytes"] / us / 1e9, 1) and r["unit"] == "GB/s"
            assert r["frac"] == round(r["achieved"] / bench.HBM_PEAK_GBS, 4)
        else:
            assert r["achieved"] == round(a["attn_flops"] / us / 1e12, 1) and r["unit"] == "TFLOP/s"
            assert r["frac"] == round(a["attn_flops"] / us / 1e12 / bench.mfma_peak_tflops(w, a), 4)
        assert r["frac_of_measured_hbm"] == round(a["decode_bytes"] / us / 1e9 / 6000.0, 4)


def test_mixed_mfma_peak():
    """Per token and query row the score product is 2 (d_c + d_r) flops and
    P . V 2 d_c; at d_c = 512, d_r = 64 the two at 5.0 and 2.5 PFLOP/s give
    1088 / (576 / 5 + 512 / 2.5) = 3400 TFLOP/s.  bf16 caches, and e4m3 with
    at most 64 query rows (decoded to bf16), stay at 2.5."""
    from workloads.generate import make_inputs
    w = get_workload("kimi_k2_fp8")
    a = bench.algorithmic(w, make_inputs(w, poison=False)["seq_lens"])
    assert a["score_flops"] + a["pv_flops"] == a["attn_flops"]
    assert a["score_flops"] * 512 == a["pv_flops"] * 576
    assert abs(bench.mfma_peak_tflops(w, a) - 3400.0) < 1e-6
    w2 = get_workload("deepseek_v3")
    assert bench.mfma_peak_tflops(w2, bench.algorithmic(w2, [4096] * 32)) == bench.MFMA_BF16_PEAK_TFLOPS
    w3 = small_workload("kimi_k2_fp8", heads=16)  # 64 rows: the few-rows kernel
    assert bench.mfma_peak_tflops(w3, bench.algorithmic(w3, [300] * w3.batch)) == bench.MFMA_BF16_PEAK_TFLOPS
