"""Pins of the TPLA oracle (latent split with an optional Hadamard change of
basis, emulated on one device) against what the mathematics fixes:

* the Hadamard matrix is orthonormal and is scipy's Sylvester construction;
* one shard is plain MLA, with or without the change of basis (full MLA is
  invariant under an orthogonal basis change of the latent);
* a latent confined to the first shard's channels makes the split exact
  (the other shards see zero latent and add nothing);
* all-zero queries give uniform attention on every shard, whose sum is the
  MLA output whatever the basis;
* planted mistakes in the oracle (interleaved channels, averaging instead of
  summing, an unrotated W_UV) break at least one of these.
"""
from dataclasses import replace

import numpy as np
import pytest
import scipy.linalg

import oracle
import oracle.tpla_oracle as tpla
from workloads import make_inputs, small_workload


def _inputs(**kw):
    w = small_workload("deepseek_v3", batch=2, heads=3, seq_len=(5, 40), max_seq_len=64, forced_lens=(40, 7), **kw)
    return make_inputs(w)


def _close(a, b, atol):
    return np.allclose(a, b, rtol=0, atol=atol)


@pytest.mark.parametrize("d", [1, 2, 4, 64, 256, 512])
def test_hadamard_is_orthonormal_sylvester(d):
    h = oracle.hadamard(d)
    assert _close(h @ h.T, np.eye(d), 1e-12)
    assert np.array_equal(h, h.T)
    assert _close(h, scipy.linalg.hadamard(d) / np.sqrt(d), 1e-15)


def test_hadamard_rejects_other_orders():
    with pytest.raises(ValueError):
        oracle.hadamard(3)


@pytest.mark.parametrize("rotate", [False, True])
def test_one_shard_is_mla(rotate):
    inp = _inputs()
    ref = oracle.decode(inp)
    got = oracle.tpla_decode(inp, 1, rotate)
    assert _close(got["out"], ref["out"], 1e-9)
    assert _close(got["shard_lse"][0], ref["lse"], 1e-9)


def _confine_to_first(inp, n):
    """Zero the latent channels of shards 1..n-1 in every record."""
    w = inp["workload"]
    cache = inp["cache"].copy()
    cache[..., w.d_latent // n: w.d_latent] = 0
    return dict(inp, cache=cache)


@pytest.mark.parametrize("n", [2, 4])
def test_latent_in_first_shard_splits_exactly(n):
    inp = _confine_to_first(_inputs(), n)
    ref = oracle.decode(inp)
    got = oracle.tpla_decode(inp, n, False)
    assert _close(got["out"], ref["out"], 1e-9)
    assert _close(got["shard_out"][1:], 0.0, 0.0)


def _zero_queries(inp):
    return dict(inp, q_nope=np.zeros_like(inp["q_nope"]), q_rope=np.zeros_like(inp["q_rope"]))


@pytest.mark.parametrize("rotate", [False, True])
def test_uniform_attention_splits_exactly(rotate):
    inp = _zero_queries(_inputs())
    ref = oracle.decode(inp)
    got = oracle.tpla_decode(inp, 2, rotate)
    assert _close(got["out"], ref["out"], 1e-9)


def test_split_is_an_approximation():
    """With informative queries two shards do not reproduce MLA: the
    emulation measures a real difference."""
    inp = _inputs()
    ref = oracle.decode(inp)["out"]
    for rotate in (False, True):
        got = oracle.tpla_decode(inp, 2, rotate)["out"]
        assert np.linalg.norm(got - ref) > 1e-3 * np.linalg.norm(ref)


# ----------------------------------------------------------- planted mistakes

def test_planted_interleaved_channels_fail(monkeypatch):
    monkeypatch.setattr(tpla, "shard_channels", lambda d, n, i: np.arange(i, d, n))
    inp = _confine_to_first(_inputs(), 2)
    got = oracle.tpla_decode(inp, 2, False)
    assert not _close(got["out"], oracle.decode(inp)["out"], 1e-6)


def test_planted_mean_instead_of_sum_fails(monkeypatch):
    monkeypatch.setattr(tpla, "aggregate", lambda s: s.mean(axis=0))
    inp = _zero_queries(_inputs())
    got = oracle.tpla_decode(inp, 2, False)
    assert not _close(got["out"], oracle.decode(inp)["out"], 1e-6)


def test_planted_unrotated_values_fail(monkeypatch):
    real = tpla.rotated

    def wrong(inputs, rotate):
        values, w_uk, _ = real(inputs, rotate)
        return values, w_uk, oracle.bf16_to_f64(inputs["w_uv"])

    monkeypatch.setattr(tpla, "rotated", wrong)
    inp = _inputs()
    got = oracle.tpla_decode(inp, 1, True)
    assert not _close(got["out"], oracle.decode(inp)["out"], 1e-6)


def test_stored_rounding_is_exact_without_rotation():
    """Without the basis change the latent and the weights are bf16 values
    already: the stored-precision model must change nothing."""
    inp = _inputs()
    a = oracle.tpla_decode(inp, 2, False)
    b = oracle.tpla_decode(inp, 2, False, stored=True)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["shard_lse"], b["shard_lse"])


def test_stored_rounding_is_nearest_bf16():
    """Every rounded value is a bf16 value within half a bf16 step of the
    exact one (8 significant bits: half a step is 2^-9 of the magnitude's
    binade), rounding twice changes nothing, and the rounded rotated decode
    stays close to the exact one."""
    inp = _inputs()
    w = inp["workload"]
    values, w_uk, _ = tpla.rotated(inp, True)
    x = np.concatenate([values[..., : w.d_latent].ravel(), w_uk.ravel()])
    x = x[np.isfinite(x)]  # unused cache slots hold NaN by construction
    r = tpla.stored_bf16(x)
    nz = x != 0
    half_step = 2.0 ** (np.floor(np.log2(np.abs(x[nz]))) - 8)
    assert np.all(np.abs(r[nz] - x[nz]) <= half_step * (1 + 1e-12))
    assert np.array_equal(tpla.stored_bf16(r), r)
    assert np.array_equal(r[~nz], x[~nz])
    exact = oracle.tpla_decode(inp, 2, True)["out"]
    kept = oracle.tpla_decode(inp, 2, True, stored=True)["out"]
    assert not np.array_equal(exact, kept)
    assert _close(exact, kept, 2e-2)
