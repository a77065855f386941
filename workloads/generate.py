"""Seeded input generation for the decode workloads.

Everything here is input preparation: random draws, the page permutation,
and the stored encodings (bf16 bits by round-to-nearest-even; OCP e4m3 bytes
with one fp32 scale per token).  No attention arithmetic lives here.

Draw recipe (one independent child stream per item, so that changing one
item's size never shifts another's values):
  SeedSequence(seed).spawn(5) -> [lengths, weights, queries, cache, pages]
  lengths : integers uniform in [lo, hi] (both ends included); ``forced_lens``
            overrides the first entries
  weights : W_UK [H, d_n, d_c] then W_UV [H, d_c, d_v], N(0, weight_var), fp32 -> bf16
  queries : q_nope [B, S_q, H, d_n] then q_rope [B, S_q, H, d_r], N(0, 1) -> bf16
  cache   : one N(0, 1) fp32 record [c_KV (d_c) | k_rope (d_r)] per token, in
            (sequence, position) order -> bf16, or -> e4m3 with scale amax/448
  pages   : a random permutation of the physical page ids (identity when the
            workload is contiguous), handed out in (sequence, logical block) order
Slots past a sequence's length in its last page, spare pages and unused
block-table entries are poisoned (NaN bits, NaN scales, -1 page ids) so that a
kernel reading them shows up in the results.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3_MAX = 448.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3 (e4m3fn) bytes, round to nearest even, after clamping to +-448."""
    import torch

    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_inputs(w: Workload, seed: int | None = None, poison: bool = True) -> dict:
    """Draw one workload's inputs.  Arrays are host numpy arrays in the
    library's device layouts (bf16 and e4m3 as raw bit patterns)."""
    seed = w.seed if seed is None else seed
    s_len, s_w, s_q, s_kv, s_pg = [np.random.default_rng(c) for c in np.random.SeedSequence(seed).spawn(5)]

    B, H, S, dn, dr, dc, dv, bs = w.batch, w.heads, w.q_len, w.d_nope, w.d_rope, w.d_latent, w.d_v, w.block_size
    lo, hi = w.seq_len
    lens = s_len.integers(lo, hi + 1, size=B, dtype=np.int64)
    for i, v in enumerate(w.forced_lens[:B]):
        lens[i] = v
    if np.any(lens > w.capacity) or np.any(lens < 0):
        raise ValueError("sequence length outside [0, capacity]")
    seq_lens = lens.astype(np.int32)

    wstd = float(np.sqrt(w.weight_var))
    w_uk = f32_to_bf16_bits(_normal(s_w, (H, dn, dc), wstd))
    w_uv = f32_to_bf16_bits(_normal(s_w, (H, dc, dv), wstd))
    q_nope = f32_to_bf16_bits(_normal(s_q, (B, S, H, dn)))
    q_rope = f32_to_bf16_bits(_normal(s_q, (B, S, H, dr)))

    # Physical pages.
    nblk = [-(-int(L) // bs) for L in lens]
    used = int(sum(nblk))
    total_blocks = max(1, used + w.spare_blocks)
    perm = s_pg.permutation(total_blocks).astype(np.int32) if w.paged else np.arange(total_blocks, dtype=np.int32)
    MB = w.max_blocks_per_seq
    block_table = np.full((B, MB), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        block_table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += nblk[b]

    # Where each (sequence, position) record lives in the flat [pages * bs] slot array.
    ntok = int(lens.sum())
    dest = np.empty(ntok, dtype=np.int64)
    pos = 0
    for b in range(B):
        L = int(lens[b])
        t = np.arange(L, dtype=np.int64)
        dest[pos: pos + L] = block_table[b, t // bs].astype(np.int64) * bs + t % bs
        pos += L

    rec = dc + dr
    values = _normal(s_kv, (ntok, rec))
    out = dict(
        workload=w, seed=seed, q_nope=q_nope, q_rope=q_rope, w_uk=w_uk, w_uv=w_uv,
        block_table=block_table, seq_lens=seq_lens, softmax_scale=w.softmax_scale,
        num_blocks=total_blocks,
    )
    if w.cache_dtype == "bf16":
        cache = np.full((total_blocks * bs, rec), BF16_NAN if poison else 0, dtype=np.uint16)
        cache[dest] = f32_to_bf16_bits(values)
        out["cache"] = cache.reshape(total_blocks, bs, rec)
        out["kv_scale"] = None
    elif w.cache_dtype == "fp8_e4m3":
        amax = np.max(np.abs(values), axis=1)
        scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        scale[amax == 0] = np.float32(1.0)
        codes = f32_to_e4m3_bits(values / scale[:, None])
        cache = np.full((total_blocks * bs, rec), E4M3_NAN if poison else 0, dtype=np.uint8)
        cache[dest] = codes
        kv_scale = np.full(total_blocks * bs, np.nan if poison else 1.0, dtype=np.float32)
        kv_scale[dest] = scale
        out["cache"] = cache.reshape(total_blocks, bs, rec)
        out["kv_scale"] = kv_scale.reshape(total_blocks, bs)
    else:
        raise ValueError(f"unknown cache dtype {w.cache_dtype!r}")
    return out


def replicate_cache(inputs: dict, n: int) -> list:
    """``n`` independent host copies of the cache (and scales); the bench
    rotates device copies so consecutive steps cannot hit in on-die caches."""
    reps = []
    for _ in range(n):
        reps.append((inputs["cache"].copy(), None if inputs["kv_scale"] is None else inputs["kv_scale"].copy()))
    return reps


def make_append_inputs(w: Workload, seed: int | None = None) -> dict:
    """Inputs of the cache append for the S_q new tokens of every sequence:
    hidden states x [B, S_q, d_model] ~ N(0, 1) and the combined projection
    [W_DKV | W_KR] [d_model, d_c + d_r] ~ N(0, 1/d_model), both as bf16 bits,
    and the RoPE base.  Drawn from child stream 5 of the workload seed (the
    decode inputs use children 0-4, so they are unchanged)."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(6)[5])
    D, B, S = w.d_model, w.batch, w.q_len
    x = f32_to_bf16_bits(_normal(rng, (B, S, D)))
    w_dkv = f32_to_bf16_bits(_normal(rng, (D, w.d_latent + w.d_rope), float(np.sqrt(1.0 / D))))
    return dict(x=x, w_dkv=w_dkv, rope_base=10000.0)


def make_prefill_inputs(w: Workload, prompt_len: int, seed: int | None = None) -> dict:
    """Inputs of an MLA-form prefill: prompts of the workload's batch padded
    to ``prompt_len`` positions, lengths drawn like the workload's (clipped to
    prompt_len, ``forced_lens`` first); the prompt's records ckr
    [B, P, d_c + d_r] and q_nope / q_rope [B, P, H, .] ~ N(0, 1), W_UK / W_UV
    ~ N(0, weight_var), all as bf16 bits.  Child stream 6 of the seed."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(7)[6])
    B, H, P = w.batch, w.heads, prompt_len
    lo, hi = w.seq_len
    lens = rng.integers(min(lo, P), min(hi, P) + 1, size=B, dtype=np.int64)
    for i, v in enumerate(w.forced_lens[:B]):
        lens[i] = min(v, P)
    wstd = float(np.sqrt(w.weight_var))
    w_uk = f32_to_bf16_bits(_normal(rng, (H, w.d_nope, w.d_latent), wstd))
    w_uv = f32_to_bf16_bits(_normal(rng, (H, w.d_latent, w.d_v), wstd))
    q_nope = f32_to_bf16_bits(_normal(rng, (B, P, H, w.d_nope)))
    q_rope = f32_to_bf16_bits(_normal(rng, (B, P, H, w.d_rope)))
    ckr = f32_to_bf16_bits(_normal(rng, (B, P, w.d_latent + w.d_rope)))
    return dict(workload=w, prompt_len=P, seq_lens=lens.astype(np.int32), w_uk=w_uk, w_uv=w_uv, q_nope=q_nope,
                q_rope=q_rope, ckr=ckr, softmax_scale=w.softmax_scale)


def make_gqa_inputs(w: Workload, groups: int, seed: int | None = None, poison: bool = True) -> dict:
    """Inputs of a GQA decode over a per-group expanded cache (the second
    decoding path of the GQLA abstract): the H heads form ``groups`` groups of
    H / groups consecutive heads; each (sequence, group) stream holds, per
    position, the record [K_nope (d_n) | V (d_v) | k_rope (d_r)], the RoPE key
    being the token's one shared key repeated in every group's record.
    Queries q_nope / q_rope [B, S_q, H, .], K_nope, V, k_rope ~ N(0, 1), bf16.
    Streams are paged like the latent cache: stream (b, g) = b * groups + g
    has its own block-table row; seq_lens [B] and per stream.  Child stream 7
    of the seed (lengths, queries, cache, pages)."""
    seed = w.seed if seed is None else seed
    if w.heads % groups:
        raise ValueError("heads must split evenly into groups")
    s_len, s_q, s_kv, s_pg = [np.random.default_rng(c) for c in np.random.SeedSequence(seed).spawn(8)[7].spawn(4)]
    B, H, S, G, bs = w.batch, w.heads, w.q_len, groups, w.block_size
    dn, dv, dr = w.d_nope, w.d_v, w.d_rope
    lo, hi = w.seq_len
    lens = s_len.integers(lo, hi + 1, size=B, dtype=np.int64)
    for i, v in enumerate(w.forced_lens[:B]):
        lens[i] = v
    if np.any(lens > w.capacity) or np.any(lens < 0):
        raise ValueError("sequence length outside [0, capacity]")
    q_nope = f32_to_bf16_bits(_normal(s_q, (B, S, H, dn)))
    q_rope = f32_to_bf16_bits(_normal(s_q, (B, S, H, dr)))
    # pages of the B * G streams
    nblk = [-(-int(lens[bg // G]) // bs) for bg in range(B * G)]
    total_blocks = max(1, int(sum(nblk)) + w.spare_blocks)
    perm = s_pg.permutation(total_blocks).astype(np.int32) if w.paged else np.arange(total_blocks, dtype=np.int32)
    MB = w.max_blocks_per_seq
    block_table = np.full((B * G, MB), -1, dtype=np.int32)
    off = 0
    for bg in range(B * G):
        block_table[bg, : nblk[bg]] = perm[off: off + nblk[bg]]
        off += nblk[bg]
    rec = dn + dv + dr
    cache = np.full((total_blocks * bs, rec), BF16_NAN if poison else 0, dtype=np.uint16)
    for b in range(B):
        L = int(lens[b])
        t = np.arange(L, dtype=np.int64)
        kr = f32_to_bf16_bits(_normal(s_kv, (L, dr)))           # one RoPE key per token
        for g in range(G):
            kv = f32_to_bf16_bits(_normal(s_kv, (L, dn + dv)))  # this group's K_nope | V
            dest = block_table[b * G + g, t // bs].astype(np.int64) * bs + t % bs
            cache[dest, : dn + dv] = kv
            cache[dest, dn + dv:] = kr
    return dict(workload=w, groups=G, q_nope=q_nope, q_rope=q_rope, seq_lens=lens.astype(np.int32),
                stream_lens=np.repeat(lens.astype(np.int32), G), block_table=block_table,
                cache=cache.reshape(total_blocks, bs, rec), num_blocks=total_blocks,
                softmax_scale=w.softmax_scale)
