"""Pins of the cache-append oracle (down-projection, RoPE, encoders, page
slots) against facts that do not come from the oracle itself.

Each pin is a ``check_*`` function taking the oracle module, so that
``test_planted_mistakes_are_caught`` can hand it a copy with a deliberate bug
and show that the pin fails.
"""
import math
import types
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle.append_oracle as ao
from workloads import Workload, f32_to_bf16_bits, make_append_inputs, make_inputs


def tiny(**kw) -> Workload:
    base = dict(name="tiny_append", batch=4, heads=2, q_len=2, d_latent=8, seq_len=(3, 13), paged=True,
                cache_dtype="bf16", out_dtype="bf16", weight_var=1.0 / 8, seed=11, d_nope=8, d_rope=4,
                d_v=8, block_size=4, spare_blocks=3, d_model=6, forced_lens=(0, 2, 4, 13))
    base.update(kw)
    return Workload(**base)


def _bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ RoPE

def check_rope_rotation_2d(m):
    """d = 2: the single pair turns by exactly pos radians (theta_0 = 1 for
    any base), counter-clockwise: the textbook rotation of (1, 0)."""
    for p in (0.0, 0.5, math.pi / 2, 3.0, 100.0):
        got = m.rope(np.array([1.0, 0.0]), p, 10000.0)
        assert np.allclose(got, [math.cos(p), math.sin(p)], atol=1e-12), (p, got)
    got = m.rope(np.array([0.0, 1.0]), math.pi / 2, 10000.0)
    assert np.allclose(got, [-1.0, 0.0], atol=1e-12)


def check_rope_complex(m):
    """Pairs (2i, 2i+1) as complex numbers z_i are multiplied by
    exp(1j * pos * base^(-2i/d)) (complex arithmetic, a second route)."""
    rng = np.random.default_rng(3)
    d, base = 16, 500.0
    v = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 123, 4096])
    z = v[:, 0::2] + 1j * v[:, 1::2]
    freq = np.power(base, -np.arange(0, d, 2) / d)
    zr = z * np.exp(1j * pos[:, None] * freq[None, :])
    want = np.empty_like(v)
    want[:, 0::2], want[:, 1::2] = zr.real, zr.imag
    assert np.allclose(m.rope(v, pos, base), want, atol=1e-9)


def check_rope_relative(m):
    """RoPE's defining property: <R(q, a), R(k, b)> depends only on a - b,
    and rotations compose: R(R(v, a), b) = R(v, a + b); norms are kept."""
    rng = np.random.default_rng(4)
    d = 64
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for a, b in ((10, 3), (5000, 4990), (0, 0), (77, 1000)):
        lhs = m.rope(q, a) @ m.rope(k, b)
        rhs = m.rope(q, a - b) @ k
        assert abs(lhs - rhs) < 1e-8 * (1 + abs(rhs)), (a, b, lhs, rhs)
        assert np.allclose(m.rope(m.rope(q, a), b), m.rope(q, a + b), atol=1e-8)
        assert abs(np.linalg.norm(m.rope(q, a)) - np.linalg.norm(q)) < 1e-10
    assert np.array_equal(m.rope(q, 0), q)


# ------------------------------------------------------------------ encoders

def check_bf16_encoder(m):
    """fp64 -> bf16 (nearest, ties to even) equals torch's fp32 -> bf16 on
    fp32 values, including exact ties."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))).astype(np.float32)
    ties = ((rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 16) | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) > 1e-30) & (np.abs(ties) < 1e38)]
    x = np.concatenate([x, ties, np.array([0.0, 1.0, -2.5], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = m.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, want), int(np.sum(got != want))


def check_e4m3_encoder(m):
    """fp64 -> OCP E4M3 (clamped to +-448, nearest, ties to even) equals
    torch's float8_e4m3fn on fp32 values across the whole range, halfway
    points and signed zeros; every finite code round-trips."""
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-14, 7, 100000))).astype(np.float32)
    vals = ao_codes_values()
    mid = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)  # exact halfway points between neighbours
    x = np.concatenate([x, mid, -mid, np.array([0.0, -0.0, 448.0, 1000.0, -1e6, 1e-9, -1e-9], np.float32)])
    want = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = m.f64_to_e4m3_bits(x.astype(np.float64))
    assert np.array_equal(got, want), int(np.sum(got != want))


def ao_codes_values():
    """The non-negative finite E4M3 values in increasing order, via torch."""
    codes = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return np.sort(codes)


# ------------------------------------------------------------------ records and slots

def check_records_brute_force(m):
    """Tiny shapes: the record of every appended token by plain Python loops
    (the product sum by sum, the rotation as complex multiplication)."""
    w = tiny()
    inp = make_inputs(w)
    ap = make_append_inputs(w)
    pos = m.append_positions(inp["seq_lens"], w.q_len)
    rec = m.append_values(ap["x"], ap["w_dkv"], w.d_latent, pos, ap["rope_base"])
    x = _bits_to_f64(ap["x"])
    W = _bits_to_f64(ap["w_dkv"])
    assert len(pos) == sum(w.q_len for L in inp["seq_lens"] if L > 0)
    for i, (b, s, p) in enumerate(pos):
        y = [sum(x[b, s, k] * W[k, n] for k in range(w.d_model)) for n in range(w.d_latent + w.d_rope)]
        lat = y[:w.d_latent]
        r = y[w.d_latent:]
        rot = []
        for j in range(w.d_rope // 2):
            z = complex(r[2 * j], r[2 * j + 1]) * complex(math.cos(p * ap["rope_base"] ** (-2 * j / w.d_rope)),
                                                          math.sin(p * ap["rope_base"] ** (-2 * j / w.d_rope)))
            rot += [z.real, z.imag]
        assert np.allclose(rec[i], lat + rot, atol=1e-12), (b, s, p)


def check_append_slots(m):
    """The append writes the last S_q positions of every live sequence, each
    to page block_table[b][pos // bs], slot pos % bs, and nothing else: every
    other slot (and scale) is unchanged bit for bit; idle slots append nothing."""
    for dtype in ("bf16", "fp8_e4m3"):
        w = tiny(cache_dtype=dtype)
        inp = make_inputs(w)
        ap = make_append_inputs(w)
        cache, scale, pos, rec = m.apply_append(inp, ap)
        want = set()
        for b, L in enumerate(int(v) for v in inp["seq_lens"]):
            for s in range(w.q_len if L > 0 else 0):
                p = L - w.q_len + s
                want.add((int(inp["block_table"][b, p // w.block_size]), p % w.block_size))
        assert {(b, s, p) for b, s, p in pos} == {(b, s, int(L) - w.q_len + s) for b, L in enumerate(inp["seq_lens"])
                                                   if L > 0 for s in range(w.q_len)}
        changed = set()
        for pg in range(cache.shape[0]):
            for sl in range(cache.shape[1]):
                if not np.array_equal(cache[pg, sl], inp["cache"][pg, sl]):
                    changed.add((pg, sl))
        assert changed <= want and len(want) == len(pos)
        bits, sc = m.encode_records(rec, dtype)
        for i, (b, s, p) in enumerate(pos):
            pg, sl = int(inp["block_table"][b, p // w.block_size]), p % w.block_size
            assert np.array_equal(cache[pg, sl], bits[i])
            if dtype != "bf16":
                assert scale[pg, sl] == np.float32(sc[i])
        if dtype != "bf16":
            others = np.ones(scale.shape, bool)
            for pg, sl in want:
                others[pg, sl] = False
            assert np.array_equal(scale[others], inp["kv_scale"][others], equal_nan=True)


def check_fp8_scale(m):
    """An e4m3 record's scale maps its largest magnitude exactly onto 448
    (code 0x7E), and the decoded record is within half a code step of
    v / scale."""
    rng = np.random.default_rng(8)
    rec = rng.standard_normal((20, 40)) * np.exp(rng.uniform(-3, 3, (20, 1)))
    codes, scale = m.encode_records(rec, "fp8_e4m3")
    assert np.allclose(scale, np.max(np.abs(rec), axis=1) / 448.0, rtol=0, atol=0)
    assert np.all(np.max(codes & 0x7F, axis=1) == 0x7E)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    y = rec / scale[:, None]
    step = np.maximum(np.ldexp(1.0, np.frexp(np.abs(y))[1] - 4), 2.0 ** -9)
    assert np.all(np.abs(vals - y) <= step / 2 + 1e-12)


PINS = [check_rope_rotation_2d, check_rope_complex, check_rope_relative, check_bf16_encoder, check_e4m3_encoder,
        check_records_brute_force, check_append_slots, check_fp8_scale]


@pytest.mark.parametrize("check", PINS, ids=[c.__name__ for c in PINS])
def test_append_oracle_pin(check):
    check(ao)


# ------------------------------------------------------------------ planted mistakes

def _mutant(**patches):
    mm = types.ModuleType("append_oracle_mutant")
    mm.__dict__.update({k: getattr(ao, k) for k in dir(ao) if not k.startswith("__")})
    for name in dir(ao):
        fn = getattr(ao, name)
        if isinstance(fn, types.FunctionType) and fn.__module__ == ao.__name__:
            mm.__dict__[name] = types.FunctionType(fn.__code__, mm.__dict__, name, fn.__defaults__, fn.__closure__)
    mm.__dict__.update(patches)
    return mm


def _rope_clockwise(v, pos, base=10000.0):
    return ao.rope(v, -np.asarray(pos, dtype=np.float64), base)


def _rope_half_pairs(v, pos, base=10000.0):  # pairs (i, i + d/2) instead of (2i, 2i+1)
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inter = np.empty_like(v)
    inter[..., perm] = v
    out = ao.rope(inter, pos, base)
    return out[..., perm]


def _rope_wrong_freq(v, pos, base=10000.0):  # base^(-i/d)
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    th = base ** (-np.arange(d // 2) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * th
    out = np.empty_like(v)
    out[..., 0::2] = v[..., 0::2] * np.cos(ang) - v[..., 1::2] * np.sin(ang)
    out[..., 1::2] = v[..., 0::2] * np.sin(ang) + v[..., 1::2] * np.cos(ang)
    return out


def _bf16_truncate(x):
    return (np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _e4m3_half_up(x):
    x = np.clip(np.asarray(x, dtype=np.float64), -448, 448)
    vals = ao_codes_values()
    a = np.abs(x)
    idx = np.searchsorted(vals, a, side="right") - 1
    idx = np.clip(idx, 0, len(vals) - 1)
    up = np.clip(idx + 1, 0, len(vals) - 1)
    pick = np.where(a - vals[idx] >= vals[up] - a, up, idx)  # ties away from zero
    codes = torch.from_numpy(vals[pick].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)


def _positions_shifted(seq_lens, q_len):
    return [(b, s, p - 1) for b, s, p in ao.append_positions(seq_lens, q_len) if p > 0]


def _no_rope_values(x_bits, w_bits, d_latent, positions, base):
    x = _bits_to_f64(x_bits)
    w = _bits_to_f64(w_bits)
    return np.stack([x[b, s] for b, s, _ in positions]) @ w


def _scale_rms(rec, cache_dtype):
    if cache_dtype == "bf16":
        return ao.f64_to_bf16_bits(rec), None
    sc = np.sqrt(np.mean(rec ** 2, axis=1)) / 448 * 8
    return ao.f64_to_e4m3_bits(rec / sc[:, None]), sc


@pytest.mark.parametrize("patch,check", [
    (dict(rope=_rope_clockwise), check_rope_rotation_2d),
    (dict(rope=_rope_clockwise), check_records_brute_force),
    (dict(rope=_rope_half_pairs), check_rope_complex),
    (dict(rope=_rope_half_pairs), check_records_brute_force),
    (dict(rope=_rope_wrong_freq), check_rope_complex),
    (dict(f64_to_bf16_bits=_bf16_truncate), check_bf16_encoder),
    (dict(f64_to_e4m3_bits=_e4m3_half_up), check_e4m3_encoder),
    (dict(append_positions=_positions_shifted), check_append_slots),
    (dict(append_values=_no_rope_values), check_records_brute_force),
    (dict(encode_records=_scale_rms), check_fp8_scale),
])
def test_planted_mistakes_are_caught(patch, check):
    with pytest.raises(AssertionError):
        check(_mutant(**patch))
