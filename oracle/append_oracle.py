"""Oracle: latent down-projection, decoupled RoPE key and paged cache append, in fp64.

TEST INFRASTRUCTURE.  Only the test suite and the bench's CPU-baseline leg use
this module; the HIP library neither imports nor calls it, and the two share
no code.

What is computed, and where the pages state it
---------------------------------------------
* A token's latent is the down-projection of its hidden state, c_KV = x W_DKV
  (the matrix the TransMLA review page calls W_DKV, Eq. (11), in
  referee_report.minor_comments), and only that latent is cached together
  with one decoupled RoPE key shared by every head (TransMLA review page,
  core_discovery; TPLA abstract on the taxoreview pages).
* The RoPE key is the projection x W_KR of the same hidden state, rotated by
  the token's position.  Both projections are taken here as one matrix
  [W_DKV | W_KR] of d_model x (d_c + d_r), latent columns first.
* The record [c_KV | k_rope] is written to the token's slot of the paged
  cache: page block_table[b][pos // block_size], slot pos % block_size.

Readings taken where the pages are silent (also listed with the design
notes): the rotation is RoPE as RoFormer defines it, pairs (2i, 2i+1) of the
d_r dimensions turned by the angle pos * base^(-2i/d_r) with base 10000; the
S_q new tokens of sequence b take the last positions L_b - S_q + s (the same
convention the decode uses for its queries); an idle slot (L_b = 0) appends
nothing; bf16 records are rounded to nearest even; an e4m3 record is the
e4m3 value (round to nearest even, after clamping to +-448) of v / scale with
one fp32 scale per token, scale = max|v| / 448 over the whole record (1 when
the record is all zeros).
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def rope(v: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate the last axis of v (even length d) by position pos: pair
    (2i, 2i+1) turns by pos * base^(-2i/d).  pos broadcasts against
    v.shape[:-1]."""
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even) and return the bit
    patterns.  bf16 keeps 8 significant bits: with |x| = f * 2^e, f in
    [0.5, 1), the representable neighbours are multiples of 2^(e-8).  Values
    must be zero or inside the normal bf16 range."""
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(f, 8)), e - 8)  # np.rint rounds half to even
    r = np.where(x == 0, 0.0, r)
    if np.any((r != 0) & (np.abs(r) < 2.0 ** -126)):
        raise ValueError("value below the normal bf16 range")
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f64_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to OCP E4M3 (e4m3fn: bias 7, 3 mantissa bits, max
    448, subnormals 2^-9 * m) after clamping to +-448, ties to even, and
    return the bytes."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a = f * 2^e, f in [0.5, 1)
    E = np.maximum(e - 1, -6)                # binade exponent; below 2^-6 the subnormal step
    q = np.ldexp(np.rint(np.ldexp(a, 3 - E)), E - 3)  # multiples of 2^(E-3), half to even
    q = np.minimum(q, E4M3_MAX)
    # encode the rounded magnitude
    _, e2 = np.frexp(q)
    E2 = e2 - 1
    normal = q >= 2.0 ** -6
    mant_n = np.where(normal, np.ldexp(q, -np.where(normal, E2, 0)) - 1.0, 0.0) * 8.0
    code_n = ((E2 + 7) << 3) + np.rint(mant_n).astype(np.int64)
    code_s = np.rint(np.ldexp(q, 9)).astype(np.int64)  # subnormal: q = m * 2^-9
    code = np.where(normal, code_n, code_s)
    code = np.where(q == 0, 0, code)
    sign = np.where(np.signbit(x), 0x80, 0)  # a negative value that rounds to zero keeps its sign
    return (code | sign).astype(np.uint8)


def append_positions(seq_lens, q_len: int):
    """(b, s, pos) of every token the append writes: the last q_len positions
    of each non-idle sequence."""
    out = []
    for b, L in enumerate(int(v) for v in seq_lens):
        if L == 0:
            continue
        for s in range(q_len):
            out.append((b, s, L - q_len + s))
    return out


def append_values(x_bits: np.ndarray, w_bits: np.ndarray, d_latent: int, positions, base: float):
    """fp64 records [c_KV | k_rope] of the listed tokens, in list order:
    y = x W on the exact bf16 inputs, then RoPE on the last d_r columns."""
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    w = (np.asarray(w_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    rows = np.stack([x[b, s] for b, s, _ in positions]) if positions else np.zeros((0, x.shape[-1]))
    y = rows @ w
    pos = np.array([p for _, _, p in positions], dtype=np.float64)
    rec = y.copy()
    rec[:, d_latent:] = rope(y[:, d_latent:], pos, base)
    return rec


def encode_records(rec: np.ndarray, cache_dtype: str):
    """Stored form of fp64 records: bf16 bits, or e4m3 bytes and the fp32 scale per record."""
    if cache_dtype == "bf16":
        return f64_to_bf16_bits(rec), None
    amax = np.max(np.abs(rec), axis=1)
    scale = np.where(amax == 0, 1.0, amax / E4M3_MAX)
    return f64_to_e4m3_bits(rec / scale[:, None]), scale


def apply_append(inputs: dict, ap: dict):
    """The cache after the append, computed on the host: a copy of the input
    cache (and scales) with the new records written to their page slots.
    Returns (cache, kv_scale, positions, records_fp64)."""
    w = inputs["workload"]
    positions = append_positions(inputs["seq_lens"], w.q_len)
    rec = append_values(ap["x"], ap["w_dkv"], w.d_latent, positions, ap["rope_base"])
    bits, scale = encode_records(rec, w.cache_dtype)
    cache = inputs["cache"].copy()
    kv_scale = None if inputs["kv_scale"] is None else inputs["kv_scale"].copy()
    bs = w.block_size
    for i, (b, _, pos) in enumerate(positions):
        page = int(inputs["block_table"][b, pos // bs])
        cache[page, pos % bs] = bits[i]
        if scale is not None:
            kv_scale[page, pos % bs] = np.float32(scale[i])
    return cache, kv_scale, positions, rec


def with_appended(inputs: dict, ap: dict) -> dict:
    """A copy of the decode inputs whose cache holds the appended records."""
    cache, kv_scale, _, _ = apply_append(inputs, ap)
    out = dict(inputs)
    out["cache"] = cache
    out["kv_scale"] = kv_scale
    return out
