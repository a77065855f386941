"""Oracle: TPLA latent-split decode emulated on one device, in fp64.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
CPU-baseline leg use this module; the HIP library neither imports nor calls
it, and the two share no code.

What is computed, and where the pages state it
---------------------------------------------
* TPLA splits the cached latent, and each head's input dimension with it,
  over n devices; every shard runs attention on its own slice and an
  all-reduce adds the shards' results.  Each head still reads the whole
  latent, spread over the shards (TPLA abstract on the taxoreview pages for
  dblp:408/6122 and dblp:256/5536-3).
* An orthogonal change of basis of the latent, a Hadamard transform among
  the forms named there, is applied before the split to reduce the
  discrepancy between the shards.  Full MLA is unchanged by it, since
  q . c = (q R) . (c R) and c W_UV = (c R)(R^T W_UV) for orthogonal R.

Readings taken where the pages are silent (each is also listed with the
design notes):
* shard i holds the contiguous latent channels [i d_c/n, (i+1) d_c/n) of
  every record and the whole RoPE key, which every shard uses in full: its
  scores are scale (q_lat[S_i] . c[S_i] + q_rope . k_rope);
* each shard normalises its own softmax over all visible positions, and the
  aggregate is the plain sum of the shards' up-projected outputs;
* R is the Sylvester-ordered Hadamard matrix of order d_c divided by
  sqrt(d_c): c' = c R, W_UK'[h] = W_UK[h] R, W_UV'[h] = R^T W_UV[h];
* the RMSNorm reparameterization that the abstract also names acts where the
  latent is produced, before it is cached; the decode reads post-norm
  latents, so it is not part of this path.
"""
from __future__ import annotations

from dataclasses import replace

import numpy as np

from .append_oracle import f64_to_bf16_bits
from .mla_oracle import _heads, bf16_to_f64, cache_values, decode_one


def hadamard(d: int) -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix of order d (a power of two):
    H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]], divided by sqrt(d)."""
    if d < 1 or d & (d - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def rotated(inputs: dict, rotate: bool):
    """fp64 (cache values, W_UK, W_UV) of the decode inputs, with the latent
    basis changed by R when ``rotate``: c' = c R, W_UK' = W_UK R, W_UV' = R^T W_UV."""
    w = inputs["workload"]
    values = cache_values(inputs).copy()
    _, _, w_uk, w_uv, _ = _heads(inputs)
    if rotate:
        r = hadamard(w.d_latent)
        values[..., : w.d_latent] = values[..., : w.d_latent] @ r
        w_uk = w_uk @ r
        w_uv = np.einsum("cd,hdv->hcv", r.T, w_uv)
    return values, w_uk, w_uv


def shard_channels(d_latent: int, n_shards: int, i: int) -> np.ndarray:
    """Latent channels held by shard i: the i-th contiguous block of d_latent / n."""
    dcs = d_latent // n_shards
    return np.arange(i * dcs, (i + 1) * dcs)


def aggregate(shard_out: np.ndarray) -> np.ndarray:
    """The all-reduce of the shards' outputs (axis 0): their sum."""
    return shard_out.sum(axis=0)


def stored_bf16(x: np.ndarray) -> np.ndarray:
    """x as it is kept in bf16 storage: rounded to the nearest bf16 value
    (ties to even), back in fp64."""
    return bf16_to_f64(f64_to_bf16_bits(x))


def tpla_decode(inputs: dict, n_shards: int, rotate: bool, batches=None, heads=None, stored: bool = False):
    """TPLA decode of every sequence (or ``batches``) and head (or ``heads``)
    with ``n_shards`` latent shards.  Returns dict(out [B, S_q, nh, d_v] summed
    over shards, shard_out [n, B, S_q, nh, d_v], shard_lse [n, B, S_q, nh]).

    With ``stored`` the rotated latent channels and weight slices are first
    rounded to bf16, the precision the cache and the weights are kept in
    (the rotated cache replaces the cached latent in place, and the shards'
    weight slices are bf16 like the weights they come from); without it the
    basis change is exact."""
    w = inputs["workload"]
    if w.d_latent % n_shards:
        raise ValueError("d_latent must split evenly")
    dcs = w.d_latent // n_shards
    values, w_uk, w_uv = rotated(inputs, rotate)
    if stored:
        values = values.copy()
        values[..., : w.d_latent] = stored_bf16(values[..., : w.d_latent])
        w_uk, w_uv = stored_bf16(w_uk), stored_bf16(w_uv)
    q_nope, q_rope, _, _, _ = _heads(inputs)
    batches = list(range(w.batch)) if batches is None else list(batches)
    nh = w.heads if heads is None else len(list(heads))
    shard_out = np.zeros((n_shards, len(batches), w.q_len, nh, w.d_v))
    shard_lse = np.zeros((n_shards, len(batches), w.q_len, nh))
    ws = replace(w, d_latent=dcs)  # the softmax scale depends on d_nope + d_rope only
    for i in range(n_shards):
        sl = shard_channels(w.d_latent, n_shards, i)
        # shard i's records: its latent channels, then the whole RoPE key
        vals_i = np.concatenate([values[..., sl], values[..., w.d_latent:]], axis=-1)
        pre = (q_nope, q_rope, w_uk[:, :, sl], w_uv[:, sl, :], ws)
        sub = dict(inputs, workload=ws)
        for j, b in enumerate(batches):
            shard_out[i, j], shard_lse[i, j], _ = decode_one(sub, b, heads, values=vals_i, _pre=pre)
    return dict(out=aggregate(shard_out), shard_out=shard_out, shard_lse=shard_lse)
