"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Small cases span several tiles, ragged tails, idle batch slots, the causal
multi-token tail, both latent widths, the e4m3 cache and several split
counts; they compare every output element and every intermediate (absorbed
query, each split partial, merged latent output, final output).  The full
workloads run in the launch configuration the bench times and are compared on
sampled sequences and heads, which the oracle computes one by one.
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
    compare("lse", to_np(st.lse), ref["lse"], tol_abs, tol_rel, finite_only=True)
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
                    finite_only=True)
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
    # 32 heads (one wave per work-group)
    "h32": small_workload("gqa7b", batch=3, seq_len=(1, 700), max_seq_len=768, forced_lens=(129, 64, 33)),
    # latent-split shard: d_c = 256, fp32 output
    "dc256": small_workload("tpla_shard", batch=2, seq_len=(40, 400), max_seq_len=512, forced_lens=(40, 300)),
    # 4-token causal tail over an e4m3 cache, 256 rows (two row groups)
    "fp8_sq4_h64": small_workload("kimi_k2_fp8", batch=3, seq_len=(4, 300), max_seq_len=384,
                                  forced_lens=(4, 170, 33)),
    # 4-token tail, 16 heads (64 rows: two waves), bf16 cache
    "bf16_sq4_h16": replace(small_workload("kimi_k2_fp8", batch=2, heads=16, seq_len=(5, 200), max_seq_len=256,
                                           forced_lens=(5, 97)), cache_dtype="bf16"),
    # an idle batch slot (seq_len 0) next to live ones
    "idle_slot": small_workload("deepseek_v3", batch=3, seq_len=(50, 300), max_seq_len=320, forced_lens=(0, 65, 0)),
    # fp8 with 32 rows (one wave) and d_c = 512
    "fp8_h32": replace(small_workload("gqa7b", batch=2, seq_len=(3, 200), max_seq_len=256, forced_lens=(3, 161)),
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
@pytest.mark.parametrize("name", ["tiny", "h128_ragged", "dc256", "fp8_sq4_h64", "idle_slot", "h32"])
def test_small_parity_fp32_partials(name, merge):
    """The same step with fp32 split partials (o_part) instead of fp16."""
    inputs = make_inputs(SMALL_CASES[name])
    _announce(f"{name}/fp32-partials/{merge}", inputs)
    st = run_step(inputs, partial="fp32", fused=MERGES[merge])
    assert str(st.o_part.dtype) == "torch.float32"
    _check_all(inputs, st)


@pytest.mark.parametrize("merge", list(MERGES))
@pytest.mark.parametrize("name", ["h128_ragged", "dc256", "fp8_sq4_h64", "h32"])
@pytest.mark.parametrize("extra_parts", [0, 1, 5])
def test_small_parity_few_splits(name, extra_parts, merge):
    """Few token parts: each part runs many tiles and spans sequence boundaries."""
    inputs = make_inputs(SMALL_CASES[name])
    B = inputs["workload"].batch
    _announce(f"{name}+{extra_parts}/{merge}", inputs)
    st = run_step(inputs, num_parts=B + extra_parts, fused=MERGES[merge])
    _check_all(inputs, st)


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
def test_full_workload_sampled(name):
    """Each named workload at full size, in the launch configuration the bench
    times; every output is checked finite and sampled (sequence, head) pairs are
    compared with the oracle."""
    w = get_workload(name)
    inputs = make_inputs(w)
    st = run_step(inputs)
    _announce(name, inputs, st)
    out, lse = to_np(st.out), to_np(st.lse)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    tol_abs, tol_rel = tolerances(w)
    rng = np.random.default_rng(7)
    bs = sorted(set([0, w.batch - 1] + rng.integers(0, w.batch, size=2).tolist()))
    heads = sorted(set([0, w.heads - 1] + rng.integers(0, w.heads, size=4).tolist()))
    values = oracle.cache_values(inputs)
    got, ref = [], []
    got_l, ref_l = [], []
    for b in bs:
        o_ref, l_ref, _ = oracle.decode_one(inputs, b, heads, values=values)
        got.append(out[b][:, heads])
        ref.append(o_ref)
        got_l.append(lse[b][:, heads])
        ref_l.append(l_ref)
    compare(f"{name} out (sampled)", np.stack(got), np.stack(ref), tol_abs, tol_rel, scaled_abs=False)
    compare(f"{name} lse (sampled)", np.stack(got_l), np.stack(ref_l), tol_abs, tol_rel)


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
