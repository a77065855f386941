"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Small cases span several tiles, ragged tails, idle batch slots, the causal
multi-token tail, both latent widths, the e4m3 cache and several split
counts; they compare every output element and every intermediate (absorbed
query, each split partial, merged latent output, final output).  The full
workloads run in the launch configuration the bench times and are compared
element by element, over the whole output and lse tensors.
"""
import math
import sys
from dataclasses import replace

import numpy as np
import pytest

import oracle
from workloads import get_workload, make_inputs, small_workload
from gpu_helpers import compare, run_step, to_np, tolerances

pytestmark = pytest.mark.gpu


def _check_all(inputs, st, check_partials=True):
    w = inputs["workload"]
    tol_abs, tol_rel = tolerances(w)
    ref = oracle.decode(inputs)
    # absorbed query (bf16 result of an fp32 accumulation)
    compare("q_lat", to_np(st.q_lat), ref["q_lat"], tol_abs, tol_rel)
    # merged latent output (written only by the separate merge) and lse
    if st.o_lat is not None:
        compare("o_lat", to_np(st.o_lat), ref["o_lat"], tol_abs, tol_rel)
    compare("lse", to_np(st.lse), ref["lse"], tol_abs, tol_rel, finite_only=True, scaled_abs=False)
    compare("out", to_np(st.out), ref["out"], tol_abs, tol_rel)
    if check_partials:
        from head_latent_attention_absorbed_amd import split_plan
        plan = split_plan(inputs["seq_lens"], st.num_parts)
        o_part, lse_part = to_np(st.o_part), to_np(st.lse_part)
        R = w.q_len * w.heads
        values = oracle.cache_values(inputs)
        used = set()
        for slot, b, t0, t1 in plan:
            o_ref, lse_ref = oracle.partial(inputs, b, t0, t1, values=values)
            compare(f"o_part[{slot}] b={b} [{t0},{t1})", o_part[slot].reshape(w.q_len, w.heads, -1), o_ref,
                    tol_abs, tol_rel)
            compare(f"lse_part[{slot}]", lse_part[slot].reshape(w.q_len, w.heads), lse_ref, tol_abs, tol_rel,
                    finite_only=True, scaled_abs=False)
            used.add(slot)
        # slots outside the plan are never written (they still hold the NaN poison)
        for slot in range(st.num_parts):
            if slot not in used:
                assert np.all(np.isnan(lse_part[slot])), f"slot {slot} written outside the plan"
    return ref


def _announce(name, inputs, st=None):
    w = inputs["workload"]
    print(f"[case] {name}: B={w.batch} H={w.heads} S_q={w.q_len} d_c={w.d_latent} cache={w.cache_dtype} "
          f"lens={list(map(int, inputs['seq_lens']))[:8]} parts={getattr(st, 'num_parts', None)}", flush=True)


SMALL_CASES = {
    # the tiny workload exactly as specified
    "tiny": get_workload("tiny"),
    # DeepSeek-V3-like heads over ragged lengths (one token, one partial tile, multi-page)
    "h128_ragged": small_workload("deepseek_v3", batch=3, seq_len=(1, 900), max_seq_len=1024,
                                  forced_lens=(1, 77, 515), spare_blocks=3),
    # 32 heads: a block table of at most one tile per two part slots, so two
    # waves split the latent columns of each single-tile part
    "h32": small_workload("gqa7b", batch=3, seq_len=(1, 700), max_seq_len=768, forced_lens=(129, 64, 33)),
    # the same lengths under a block table with room for 8192 tokens: one wave
    # per work-group, which issues the copies and both products itself
    "h32_roomy": small_workload("gqa7b", batch=3, seq_len=(1, 700), max_seq_len=8192, forced_lens=(129, 64, 33)),
    # latent-split shard: d_c = 256, fp32 output
    "dc256": small_workload("tpla_shard", batch=2, seq_len=(40, 400), max_seq_len=512, forced_lens=(40, 300)),
    # d_c = 256 with odd tile counts (4 and 15, the last tiles partial): parts
    # that end on a pair with one tile
    "dc256_odd": small_workload("tpla_shard", batch=2, seq_len=(97, 451), max_seq_len=512, forced_lens=(97, 451)),
    # d_c = 256, two query tokens over 64 heads (128 rows): the causal tail
    # inside a pair of tiles
    "dc256_sq2_h64": small_workload("tpla_shard", batch=2, heads=64, q_len=2, seq_len=(2, 300), max_seq_len=320,
                                    forced_lens=(2, 289)),
    # 4-token causal tail over an e4m3 cache, 256 rows (two row groups)
    "fp8_sq4_h64": small_workload("kimi_k2_fp8", batch=3, seq_len=(4, 300), max_seq_len=384,
                                  forced_lens=(4, 170, 33)),
    # 4-token tail, 16 heads (64 rows: two waves), bf16 cache
    "bf16_sq4_h16": replace(small_workload("kimi_k2_fp8", batch=2, heads=16, seq_len=(5, 200), max_seq_len=256,
                                           forced_lens=(5, 97)), cache_dtype="bf16"),
    # an idle batch slot (seq_len 0) next to live ones
    "idle_slot": small_workload("deepseek_v3", batch=3, seq_len=(50, 300), max_seq_len=320, forced_lens=(0, 65, 0)),
    # fp8 with 32 rows (two column-split waves) and d_c = 512
    "fp8_h32": replace(small_workload("gqa7b", batch=2, seq_len=(3, 200), max_seq_len=256, forced_lens=(3, 161)),
                       cache_dtype="fp8_e4m3"),
    # 3-token tail over 40 heads, bf16: 120 rows, one 128-row group with 8 rows past the end
    "bf16_sq3_h40": replace(small_workload("kimi_k2_fp8", batch=2, heads=40, seq_len=(3, 300), max_seq_len=320,
                                           forced_lens=(3, 290)), q_len=3, cache_dtype="bf16"),
    # 4-token tail over 40 heads, e4m3: 160 rows, the second 128-row group 32 rows deep
    "fp8_sq4_h40": small_workload("kimi_k2_fp8", batch=2, heads=40, seq_len=(4, 300), max_seq_len=320,
                                  forced_lens=(4, 257)),
    # pages of 32, 128 and 256 records (power-of-two page sizes >= one tile)
    # through the 128-row bf16 kernel, the 128-row e4m3 kernel and the
    # few-rows kernel
    "h128_bs32": small_workload("deepseek_v3", batch=3, seq_len=(1, 900), max_seq_len=1024, block_size=32,
                                forced_lens=(900, 33, 417)),
    "h128_bs128": small_workload("deepseek_v3", batch=3, seq_len=(1, 900), max_seq_len=1024, block_size=128,
                                 forced_lens=(129, 800, 5)),
    "fp8_sq4_h64_bs128": small_workload("kimi_k2_fp8", batch=2, seq_len=(4, 600), max_seq_len=640, block_size=128,
                                        forced_lens=(600, 131)),
    "h32_bs256": small_workload("gqa7b", batch=3, seq_len=(1, 700), max_seq_len=768, block_size=256,
                                forced_lens=(700, 257, 40)),
    # e4m3 at d_c = 256 with 128 rows (2-token tail over 64 heads): the 128-row
    # e4m3 kernel's five 64-deep score steps
    "fp8_dc256_sq2_h64": replace(small_workload("tpla_shard", batch=2, heads=64, q_len=2, seq_len=(2, 300),
                                                max_seq_len=320, forced_lens=(2, 299)),
                                 cache_dtype="fp8_e4m3"),
}


MERGES = {"fused": True, "separate": False}


@pytest.mark.parametrize("merge", list(MERGES))
@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_small_parity_default_split(name, merge):
    inputs = make_inputs(SMALL_CASES[name])
    _announce(f"{name}/{merge}", inputs)
    st = run_step(inputs, fused=MERGES[merge])
    assert st.fused == MERGES[merge]
    _check_all(inputs, st)


@pytest.mark.parametrize("merge", list(MERGES))
@pytest.mark.parametrize("name", ["tiny", "h128_ragged", "dc256", "fp8_sq4_h64", "idle_slot", "h32", "h32_roomy"])
def test_small_parity_fp32_partials(name, merge):
    """The same step with fp32 split partials (o_part) instead of fp16."""
    inputs = make_inputs(SMALL_CASES[name])
    _announce(f"{name}/fp32-partials/{merge}", inputs)
    st = run_step(inputs, partial="fp32", fused=MERGES[merge])
    assert str(st.o_part.dtype) == "torch.float32"
    _check_all(inputs, st)


@pytest.mark.parametrize("merge", list(MERGES))
@pytest.mark.parametrize("name", ["h128_ragged", "dc256", "dc256_odd", "dc256_sq2_h64", "fp8_sq4_h64", "fp8_dc256_sq2_h64",
                                  "h32", "h128_bs32", "fp8_sq4_h64_bs128"])
@pytest.mark.parametrize("extra_parts", [0, 1, 5])
def test_small_parity_few_splits(name, extra_parts, merge):
    """Few token parts: each part runs many tiles (num_parts = B gives one
    part per sequence, its whole length)."""
    inputs = make_inputs(SMALL_CASES[name])
    B = inputs["workload"].batch
    _announce(f"{name}+{extra_parts}/{merge}", inputs)
    st = run_step(inputs, num_parts=B + extra_parts, fused=MERGES[merge])
    _check_all(inputs, st)


def _scale_sequence(inputs, b, e):
    """Sequence b's queries times 2^e and its cache's per-token scales times
    2^-e (both exact): the scores, softmax weights and lse stay as they were,
    the outputs scale by 2^-e."""
    w = inputs["workload"]
    f = np.float32(2.0 ** e)
    for key in ("q_nope", "q_rope"):
        x = oracle.bf16_to_f64(inputs[key][b]).astype(np.float32) * f
        inputs[key][b] = (x.view(np.uint32) >> 16).astype(np.uint16)  # exact: a power-of-two factor
    pages = inputs["block_table"][b][inputs["block_table"][b] >= 0]
    inputs["kv_scale"][pages] *= np.float32(2.0 ** -e)
    return inputs


@pytest.mark.parametrize("merge", list(MERGES))
def test_fp8_query_magnitude_range(merge):
    """e4m3 cache with query rows far outside e4m3's range: one sequence's
    queries times 2^12 (|q_lat| up to ~9e3, where e4m3 saturates at 448),
    the other's times 2^-12 (|q_lat| ~ 5e-4, below e4m3's smallest
    subnormal), each with the inverse factor on its cache scales so that the
    attention is unchanged.  The 128-row kernel splits each query row into
    e4m3 parts under a per-row power-of-two scale, so every result must equal
    the unscaled run's bit for bit after the same power of two (lse
    unchanged); the unscaled run is checked against the oracle."""
    import torch

    w = small_workload("kimi_k2_fp8", batch=2, heads=64, q_len=2, seq_len=(40, 300), max_seq_len=320,
                       forced_lens=(300, 77))
    base = make_inputs(w)
    _announce(f"fp8_query_magnitude_range/unscaled/{merge}", base)
    st0 = run_step(base, partial="fp32", fused=MERGES[merge])
    _check_all(base, st0)
    exps = (12, -12)
    scaled = make_inputs(w)
    for b, e in enumerate(exps):
        _scale_sequence(scaled, b, e)
    _announce(f"fp8_query_magnitude_range/scaled/{merge}", scaled)
    st1 = run_step(scaled, partial="fp32", fused=MERGES[merge])

    def same(name, got, ref, factor):
        got, ref = got.double().cpu(), ref.double().cpu() * factor
        ok = torch.equal(torch.nan_to_num(got, nan=7.0), torch.nan_to_num(ref, nan=7.0))
        assert ok, f"{name}: max |diff| {float((got - ref).abs().nan_to_num(0.0).max()):.3e}"

    from head_latent_attention_absorbed_amd import split_plan
    for b, e in enumerate(exps):
        same(f"q_lat[{b}]", st1.q_lat[b], st0.q_lat[b], 2.0 ** e)
        same(f"out[{b}]", st1.out[b], st0.out[b], 2.0 ** -e)
        if st0.o_lat is not None:
            same(f"o_lat[{b}]", st1.o_lat[b], st0.o_lat[b], 2.0 ** -e)
    same("lse", st1.lse, st0.lse, 1.0)
    same("lse_part", st1.lse_part, st0.lse_part, 1.0)
    for slot, b, _, _ in split_plan(base["seq_lens"], st0.num_parts):
        same(f"o_part[{slot}]", st1.o_part[slot], st0.o_part[slot], 2.0 ** -exps[b])


# Row tiles of the fused merge: 16 query rows (b*S_q + s) per work-group, so
# B*S_q = 17 and 33 leave a ragged last tile of one row, 40 one of eight.
RAGGED_ROWS = {
    "rows17": small_workload("deepseek_v3", batch=17, heads=8, seq_len=(1, 160), max_seq_len=192,
                             forced_lens=(0, 1, 33, 160)),
    "rows33_dc256": small_workload("tpla_shard", batch=33, heads=8, seq_len=(1, 100), max_seq_len=128,
                                   forced_lens=(100, 0, 2)),
    "rows40_sq4": replace(small_workload("kimi_k2_fp8", batch=10, heads=8, seq_len=(4, 120), max_seq_len=128,
                                         forced_lens=(4, 0, 120)), cache_dtype="bf16"),
}


@pytest.mark.parametrize("partial", ["fp16", "fp32"])
@pytest.mark.parametrize("name", list(RAGGED_ROWS))
def test_fused_ragged_row_tiles(name, partial):
    """The fused merge + up-projection with a partly filled last row tile,
    idle slots and one-token sequences, against the oracle and against the
    separate merge and up-projection of the same partials."""
    inputs = make_inputs(RAGGED_ROWS[name])
    _announce(f"{name}/{partial}", inputs)
    fused = run_step(inputs, partial=partial, fused=True)
    _check_all(inputs, fused)
    sep = run_step(inputs, partial=partial, fused=False)
    # same decode kernel, same partials: identical inputs to the two merges
    assert np.array_equal(to_np(fused.o_part), to_np(sep.o_part), equal_nan=True)
    tol_abs, tol_rel = tolerances(inputs["workload"])
    compare("fused vs separate out", to_np(fused.out), to_np(sep.out), tol_abs / 4, tol_rel / 4)
    compare("fused vs separate lse", to_np(fused.lse), to_np(sep.lse), 1e-5, 1e-6, finite_only=True)


@pytest.mark.parametrize("merge", list(MERGES))
def test_bitwise_deterministic(merge):
    inputs = make_inputs(SMALL_CASES["h128_ragged"])
    outs = []
    for _ in range(3):
        st = run_step(inputs, fused=MERGES[merge])
        outs.append((to_np(st.out), to_np(st.lse), to_np(st.o_part)))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b, equal_nan=True)


FULL = ["tiny", "deepseek_v3", "gqa7b", "tpla_shard", "kimi_k2_fp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload(name):
    """Each named workload at full size, in the launch configuration the bench
    times: every output element and every lse against the oracle's explicit
    reconstruction, max |err| and relative L2 over the whole tensors at the
    plain bounds (twice them for the e4m3 cache)."""
    w = get_workload(name)
    inputs = make_inputs(w)
    st = run_step(inputs)
    _announce(name, inputs, st)
    out, lse = to_np(st.out), to_np(st.lse)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    tol_abs, tol_rel = tolerances(w)
    ref = oracle.decode(inputs)
    err, rel = compare(f"{name} out", out, ref["out"], tol_abs, tol_rel, scaled_abs=False)
    lerr, lrel = compare(f"{name} lse", lse, ref["lse"], tol_abs, tol_rel, scaled_abs=False)
    print(f"[result] {name}: out max|err| {err:.3e} relL2 {rel:.3e}; lse max|err| {lerr:.3e} relL2 {lrel:.3e}",
          flush=True)


# Parts of more than 128 tiles make the one- and two-wave decode refill its
# table of tile sources in LDS (128 tiles per fill) inside the tile loop.
REFILL = {
    "h32_long": small_workload("gqa7b", batch=2, seq_len=(4500, 5000), max_seq_len=5120, forced_lens=(5000, 4500)),
    "fp8_h32_long": replace(small_workload("gqa7b", batch=2, seq_len=(4500, 5000), max_seq_len=5120,
                                           forced_lens=(5000, 4333)), cache_dtype="fp8_e4m3"),
    "h16_sq4_long": replace(small_workload("kimi_k2_fp8", batch=2, heads=16, seq_len=(4500, 5000), max_seq_len=5120,
                                           forced_lens=(4999, 4100)), cache_dtype="bf16"),
}


@pytest.mark.parametrize("extra_parts", [0, 1])
@pytest.mark.parametrize("name", list(REFILL))
def test_long_parts_refill_tile_table(name, extra_parts):
    """num_parts = B (one part per sequence, 157 tiles) and B + 1 (W = 141):
    every part crosses at least one refill of the tile-source table."""
    from head_latent_attention_absorbed_amd import split_plan

    inputs = make_inputs(REFILL[name])
    B = inputs["workload"].batch
    plan = split_plan(inputs["seq_lens"], B + extra_parts)
    assert max((t1 - t0 + 31) // 32 for _, _, t0, t1 in plan) > 128
    _announce(f"{name}+{extra_parts}", inputs)
    st = run_step(inputs, num_parts=B + extra_parts)
    _check_all(inputs, st)


def test_graph_replay_matches_eager():
    """The step captured as a HIP graph: several replays, with eager steps and
    synchronisations between them, each equal bit for bit to the eager result
    (the kernels are deterministic) and within tolerance of the oracle."""
    import torch

    inputs = make_inputs(SMALL_CASES["h128_ragged"])
    _announce("graph", inputs)
    eager = run_step(inputs)
    ref_out = to_np(eager.out)
    from head_latent_attention_absorbed_amd import DecodeStep

    st = DecodeStep(inputs)
    st.capture()
    other = DecodeStep(inputs)
    for i in range(3):
        st.out.fill_(float("nan"))
        st.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(st.out), ref_out), f"replay {i} differs from the eager step"
        other.run()  # eager work between replays
        torch.cuda.synchronize()
    tol_abs, tol_rel = tolerances(inputs["workload"])
    compare("graph out", to_np(st.out), oracle.decode(inputs)["out"], tol_abs, tol_rel)


def test_multi_step_graph_matches_eager():
    """Three steps over different inputs (as consecutive layers would be)
    captured in one graph: every replay equals each step's eager result bit
    for bit, with eager work and synchronisations between the replays."""
    import torch
    from head_latent_attention_absorbed_amd import DecodeStep, capture_steps

    cases = [SMALL_CASES["h128_ragged"], SMALL_CASES["dc256"], SMALL_CASES["fp8_sq4_h64"]]
    inputs = [make_inputs(w) for w in cases]
    _announce("multi-step graph", inputs[0])
    refs = [to_np(run_step(i).out) for i in inputs]
    steps = [DecodeStep(i) for i in inputs]
    graph = capture_steps(steps)
    other = DecodeStep(inputs[0])
    for rep in range(3):
        for st in steps:
            st.out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for j, st in enumerate(steps):
            assert np.array_equal(to_np(st.out), refs[j]), f"replay {rep}, step {j} differs from the eager step"
        other.run()
        torch.cuda.synchronize()
