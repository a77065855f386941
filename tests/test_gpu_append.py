"""Parity of the cache append (mla_append_kv, through the C ABI) with the fp64 oracle.

Cases cover one and four new tokens per sequence, idle slots, appends that
land on the last slot of a page and on the first slot of the next, both
latent widths, both cache types and a wider hidden state.  The records are
compared value by value with the oracle's (within one step of the stored
format), every other slot of the cache must be untouched bit for bit, and a
decode over the appended cache is compared with the oracle's decode of the
cache the oracle appended to.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from workloads import get_workload, make_append_inputs, make_inputs, small_workload
from gpu_helpers import compare, to_np, tolerances

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_sq1": small_workload("deepseek_v3", batch=5, seq_len=(2, 300), max_seq_len=320,
                               forced_lens=(0, 1, 64, 65, 300)),
    "bf16_sq4_h16": replace(small_workload("kimi_k2_fp8", batch=4, heads=16, seq_len=(4, 200), max_seq_len=256,
                                           forced_lens=(4, 0, 66, 131)), cache_dtype="bf16"),
    "dc256": small_workload("tpla_shard", batch=3, seq_len=(40, 400), max_seq_len=512, forced_lens=(40, 0, 257)),
    "fp8_sq4": small_workload("kimi_k2_fp8", batch=4, heads=16, seq_len=(4, 200), max_seq_len=256,
                              forced_lens=(4, 0, 64, 131)),
    "fp8_sq1": replace(small_workload("deepseek_v3", batch=3, seq_len=(2, 200), max_seq_len=256,
                                      forced_lens=(129, 0, 64)), cache_dtype="fp8_e4m3"),
    "d_model_7168": replace(small_workload("deepseek_v3", batch=3, seq_len=(2, 200), max_seq_len=256,
                                           forced_lens=(1, 128, 33)), d_model=7168),
}


def _announce(name, inputs):
    w = inputs["workload"]
    print(f"[case] append {name}: B={w.batch} S_q={w.q_len} d_c={w.d_latent} D={w.d_model} cache={w.cache_dtype} "
          f"lens={list(map(int, inputs['seq_lens']))[:8]}", flush=True)


def _host_cache(st):
    import torch

    if st.cache.dtype == torch.bfloat16:
        return st.cache.view(torch.int16).cpu().numpy().view(np.uint16)
    return st.cache.cpu().numpy()


def _append_on_device(inputs, ap):
    import torch
    from head_latent_attention_absorbed_amd import DecodeStep

    st = DecodeStep(inputs)
    st.set_append_inputs(ap)
    st.append()
    torch.cuda.synchronize()
    return st


def _e4m3_step(y):
    """Spacing of E4M3 values around |y| (subnormal spacing 2^-9 below 2^-6)."""
    a = np.abs(y)
    return np.where(a < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, np.frexp(a)[1] - 4))


@pytest.mark.parametrize("name", list(CASES))
def test_append_records(name):
    w = CASES[name]
    inputs = make_inputs(w)
    ap = make_append_inputs(w)
    _announce(name, inputs)
    st = _append_on_device(inputs, ap)
    got = _host_cache(st)
    _, _, positions, rec = oracle.apply_append(inputs, ap)
    bs = w.block_size
    slots = {(int(inputs["block_table"][b, p // bs]), p % bs): i for i, (b, _, p) in enumerate(positions)}
    assert len(slots) == len(positions) == sum(w.q_len for L in inputs["seq_lens"] if L > 0)
    # every slot the append does not own is untouched, bit for bit
    mask = np.ones(got.shape[:2], bool)
    for pg, sl in slots:
        mask[pg, sl] = False
    assert np.array_equal(got[mask], inputs["cache"][mask]), "append wrote outside the new tokens' slots"
    idx = [slots[k] for k in sorted(slots)]
    pg_sl = sorted(slots)
    rows = np.stack([got[pg, sl] for pg, sl in pg_sl])
    ref = rec[idx]
    if w.cache_dtype == "bf16":
        vals = oracle.bf16_to_f64(rows)
        err = np.abs(vals - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6), f"max err {err.max():.3e}"
        same = np.mean(rows == oracle.f64_to_bf16_bits(ref))
        assert same > 0.99, f"only {same:.4f} of the bf16 values equal the oracle's rounding"
    else:
        sc_got = to_np(st.kv_scale)
        assert np.array_equal(sc_got[mask], inputs["kv_scale"][mask], equal_nan=True), "scale written outside"
        scale = np.array([sc_got[pg, sl] for pg, sl in pg_sl])
        ref_scale = np.max(np.abs(ref), axis=1) / 448.0
        assert np.allclose(scale, ref_scale, rtol=1e-5, atol=0)
        vals = oracle.e4m3_to_f64(rows)
        y = ref / ref_scale[:, None]
        err = np.abs(vals - y)
        assert np.all(err <= _e4m3_step(y) + 1e-9), f"max err {err.max():.3e} code steps"
        same = np.mean(rows == oracle.f64_to_e4m3_bits(y))
        assert same > 0.99, f"only {same:.4f} of the e4m3 codes equal the oracle's rounding"


@pytest.mark.parametrize("name", ["bf16_sq1", "fp8_sq4", "dc256"])
def test_append_then_decode(name):
    """Append on the device, then the decode step over the appended cache,
    against the oracle's decode of the cache the oracle appended to."""
    import torch

    w = CASES[name]
    inputs = make_inputs(w)
    ap = make_append_inputs(w)
    _announce(name + "/decode", inputs)
    st = _append_on_device(inputs, ap)
    st.run()
    torch.cuda.synchronize()
    ref = oracle.decode(oracle.with_appended(inputs, ap))
    tol_abs, tol_rel = tolerances(w)
    compare("out", to_np(st.out), ref["out"], tol_abs, tol_rel)
    compare("lse", to_np(st.lse), ref["lse"], tol_abs, tol_rel, finite_only=True)


def test_append_full_workload_sampled():
    """The headline workload's shape (B = 32, d_model 4096): records of a
    sample of sequences against the oracle, the rest checked finite."""
    w = get_workload("deepseek_v3")
    inputs = make_inputs(w)
    ap = make_append_inputs(w)
    _announce("deepseek_v3", inputs)
    st = _append_on_device(inputs, ap)
    got = _host_cache(st)
    bs = w.block_size
    sample = [0, 7, 31]
    sub = dict(inputs)
    lens = np.zeros_like(inputs["seq_lens"])
    lens[sample] = inputs["seq_lens"][sample]
    sub["seq_lens"] = lens
    _, _, positions, rec = oracle.apply_append(sub, ap)
    for i, (b, _, p) in enumerate(positions):
        vals = oracle.bf16_to_f64(got[int(inputs["block_table"][b, p // bs]), p % bs])
        assert np.all(np.abs(vals - rec[i]) <= 2.0 ** -8 * np.abs(rec[i]) + 1e-6), (b, p)
    for b, L in enumerate(int(v) for v in inputs["seq_lens"]):
        vals = oracle.bf16_to_f64(got[int(inputs["block_table"][b, (L - 1) // bs]), (L - 1) % bs])
        assert np.all(np.isfinite(vals))
