"""Parity of the TPLA latent split run on one device (mla_tpla_split_weights,
mla_tpla_rotate_cache, per-shard absorb / decode / merge + up-projection,
mla_tpla_reduce, all through the C ABI) with the fp64 oracle.

The weight slices and the rotated cache are compared value by value with the
oracle's (within one bf16 rounding of an fp32 transform); the summed output
with the oracle's TPLA decode at the decode's tolerances; and a one-shard
split without the basis change must reproduce the ordinary decode bit for bit.
"""
import numpy as np
import pytest

import oracle
from workloads import get_workload, make_inputs, small_workload
from gpu_helpers import compare, to_np, tolerances

pytestmark = pytest.mark.gpu

SMALL = small_workload("deepseek_v3", batch=4, heads=16, seq_len=(1, 300), max_seq_len=320,
                       forced_lens=(300, 1, 0, 129))


def _step(inputs, n, hadamard, prepare=True):
    import torch
    from head_latent_attention_absorbed_amd import TplaStep

    st = TplaStep(inputs, n_shards=n, hadamard=hadamard)
    if prepare:
        st.prepare()
    torch.cuda.synchronize()
    return st


def _bf16_close(got_bits, ref, name):
    """Every value within half a bf16 step (plus fp32 slack) of the exact
    transform, and nearly all equal to its round-to-nearest-even."""
    got = oracle.bf16_to_f64(got_bits)
    err = np.abs(got - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-7), f"{name}: max err {err.max():.3e}"
    same = np.mean(got_bits == oracle.f64_to_bf16_bits(ref))
    assert same > 0.99, f"{name}: only {same:.4f} equal to the oracle's rounding"


def _bits(t):
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,hadamard,base", [(2, True, "deepseek_v3"), (2, False, "deepseek_v3"),
                                             (4, True, "deepseek_v3"), (1, True, "deepseek_v3"),
                                             (2, True, "tpla_shard")])
def test_split_weights(n, hadamard, base):
    """Through the entry point itself, so that shard widths without a decode
    kernel (128 of a 512 latent) are covered too."""
    import torch
    from head_latent_attention_absorbed_amd import DecodeStep, mla_tpla_split_weights

    w = small_workload(base, batch=2, heads=8, seq_len=(1, 64), max_seq_len=64)
    inputs = make_inputs(w)
    print(f"[case] tpla split weights {base} n={n} hadamard={hadamard}", flush=True)
    dec = DecodeStep(inputs)
    dcs = w.d_latent // n
    uk = torch.empty((n, w.heads, w.d_nope, dcs), dtype=torch.bfloat16, device="cuda")
    uv = torch.empty((n, w.heads, dcs, w.d_v), dtype=torch.bfloat16, device="cuda")
    mla_tpla_split_weights(dec.shape, n, hadamard, dec.w_uk, dec.w_uv, uk, uv)
    torch.cuda.synchronize()
    _, w_uk, w_uv = oracle.rotated(inputs, hadamard)
    for i in range(n):
        ch = oracle.shard_channels(w.d_latent, n, i)
        _bf16_close(_bits(uk[i]), w_uk[:, :, ch], f"w_uk shard {i}")
        _bf16_close(_bits(uv[i]), w_uv[:, ch, :], f"w_uv shard {i}")
    if not hadamard:
        assert np.array_equal(np.concatenate([_bits(uk[i]) for i in range(n)], axis=2), inputs["w_uk"])
        assert np.array_equal(np.concatenate([_bits(uv[i]) for i in range(n)], axis=1), inputs["w_uv"])


def test_rotate_cache():
    inputs = make_inputs(SMALL)
    print("[case] tpla rotate cache", flush=True)
    st = _step(inputs, 2, True)
    got = _bits(st.base.cache)
    values, _, _ = oracle.rotated(inputs, True)
    w = SMALL
    used = np.zeros(got.shape[:2], bool)
    for b, L in enumerate(int(v) for v in inputs["seq_lens"]):
        t = np.arange(L)
        used[inputs["block_table"][b, t // w.block_size], t % w.block_size] = True
    _bf16_close(got[used][:, : w.d_latent], values[used][:, : w.d_latent], "rotated latent")
    assert np.array_equal(got[..., w.d_latent:], inputs["cache"][..., w.d_latent:]), "RoPE keys changed"


@pytest.mark.parametrize("n,hadamard", [(2, True), (2, False), (1, True)])
def test_tpla_decode(n, hadamard):
    import torch

    inputs = make_inputs(SMALL)
    print(f"[case] tpla decode n={n} hadamard={hadamard} lens={list(inputs['seq_lens'])}", flush=True)
    st = _step(inputs, n, hadamard)
    st.run()
    torch.cuda.synchronize()
    ref = oracle.tpla_decode(inputs, n, hadamard)
    tol_abs, tol_rel = tolerances(SMALL)
    # the rotated cache and weights are rounded to bf16 once more than the
    # plain decode's inputs: twice the decode's bounds
    compare("out", to_np(st.out), ref["out"], 2 * tol_abs, 2 * tol_rel)
    parts = to_np(st.parts)
    for i in range(n):
        compare(f"shard {i} out", parts[i], ref["shard_out"][i], 2 * tol_abs, 2 * tol_rel)
        compare(f"shard {i} lse", to_np(st.shard_lse[i]), ref["shard_lse"][i], 2 * tol_abs, 2 * tol_rel,
                finite_only=True)


@pytest.mark.parametrize("hadamard", [True, False])
def test_tpla_decode_against_stored_model(hadamard):
    """The tighter companion check: against the oracle's TPLA decode on the
    rotated latent and weight slices rounded to bf16 (the precision the path
    keeps them in), the summed output and every shard meet the plain decode's
    bounds, not twice them."""
    import torch

    n = 2
    inputs = make_inputs(SMALL)
    print(f"[case] tpla decode stored model n={n} hadamard={hadamard}", flush=True)
    st = _step(inputs, n, hadamard)
    st.run()
    torch.cuda.synchronize()
    ref = oracle.tpla_decode(inputs, n, hadamard, stored=True)
    tol_abs, tol_rel = tolerances(SMALL)
    compare("out", to_np(st.out), ref["out"], tol_abs, tol_rel)
    parts = to_np(st.parts)
    for i in range(n):
        compare(f"shard {i} out", parts[i], ref["shard_out"][i], tol_abs, tol_rel)
        compare(f"shard {i} lse", to_np(st.shard_lse[i]), ref["shard_lse"][i], tol_abs, tol_rel, finite_only=True)


def test_one_plain_shard_is_the_decode():
    """n = 1 without the basis change runs the decode's own kernels on the same
    values: the result must match the fused decode step bit for bit."""
    import torch
    from head_latent_attention_absorbed_amd import DecodeStep

    inputs = make_inputs(SMALL)
    print("[case] tpla n=1 plain vs decode", flush=True)
    st = _step(inputs, 1, False)
    st.run()
    dec = DecodeStep(inputs, fused=True)
    dec.absorb()
    dec.decode()
    dec.combine_up()
    torch.cuda.synchronize()
    assert torch.equal(st.out.view(torch.int16), dec.out.view(torch.int16))


def test_tpla_headline_sampled():
    """The headline decode workload (B = 32, H = 128, d_c = 512, 4K-8K
    context) split in two Hadamard-basis shards: sampled sequences and heads
    against the oracle, every output finite."""
    import torch

    w = get_workload("deepseek_v3")
    inputs = make_inputs(w)
    print("[case] tpla headline sampled", flush=True)
    st = _step(inputs, 2, True)
    st.run()
    torch.cuda.synchronize()
    out = to_np(st.out)
    assert np.all(np.isfinite(out))
    batches, heads = [0, 17, 31], [0, 64, 127]
    ref = oracle.tpla_decode(inputs, 2, True, batches=batches, heads=heads)
    tol_abs, tol_rel = tolerances(w)
    compare("out sampled", out[batches][:, :, heads], ref["out"], 2 * tol_abs, 2 * tol_rel)


def test_tpla_fp8_cache_plain_split():
    """The split in the plain basis over an e4m3 cache (per-token scales apply
    to the whole record, so every shard's slice keeps its token's scale)."""
    import torch

    w = small_workload("kimi_k2_fp8", batch=3, heads=16, seq_len=(4, 200), max_seq_len=256, forced_lens=(200, 4, 0))
    inputs = make_inputs(w)
    print(f"[case] tpla fp8 plain lens={list(inputs['seq_lens'])}", flush=True)
    st = _step(inputs, 2, False)
    st.run()
    torch.cuda.synchronize()
    ref = oracle.tpla_decode(inputs, 2, False)
    tol_abs, tol_rel = tolerances(w)
    compare("out", to_np(st.out), ref["out"], 2 * tol_abs, 2 * tol_rel)
