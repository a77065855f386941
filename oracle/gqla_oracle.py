"""Oracle: GQLA's GQA decoding path over a per-group expanded cache, in fp64.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
CPU-baseline leg use this module; the HIP library neither imports nor calls
it, and the two share no code.

What is computed, and where the pages state it
---------------------------------------------
* GQLA modifies MLA so that one set of weights exposes two algebraically
  equivalent decoding paths: MLA's absorbed MQA path over the latent, and a
  GQA path over a cache expanded per head group; the GQA path is the one run
  with two query tokens per step (s_q = 2) where it suits the hardware (GQLA
  abstract on the "GQA-to-MLA" Daily Papers listing).
* Equivalence requires the heads of a group to share their up-projections:
  the group's keys K_g = W_UK[g] c and values V_g = c W_UV[g] are then what
  every head of the group reconstructs, so GQA attention over (K_g, V_g)
  equals the absorbed decode with W_UK[h] = W_UK[g(h)], W_UV[h] = W_UV[g(h)].

Readings taken where the pages are silent (also listed with the design
notes): groups are runs of H / G consecutive heads (head h is in group
h // (H / G)); the decoupled RoPE key stays one per token, shared by all
groups; query s of an S_q-token step sees positions t <= L - S_q + s, as in
the absorbed decode.
"""
from __future__ import annotations

import math

import numpy as np

from .mla_oracle import attend, bf16_to_f64, visible_limit


def group_of(h: int, heads: int, groups: int) -> int:
    """The group head h belongs to: runs of heads / groups consecutive heads."""
    return h // (heads // groups)


def gqa_stream(gi: dict, b: int, g: int, values: np.ndarray | None = None):
    """Stream (b, g)'s records in position order: K_nope [L, d_n], V [L, d_v],
    k_rope [L, d_r].  Position t of stream s = b * G + g lives in page
    block_table[s][t // block] at slot t % block.  ``values``: fp64 records
    to read instead of the stored bf16 cache (same page layout)."""
    w = gi["workload"]
    G = gi["groups"]
    L = int(gi["seq_lens"][b])
    t = np.arange(L)
    pages = gi["block_table"][b * G + g, t // w.block_size]
    src = values if values is not None else gi["cache"]
    rec = src[pages, t % w.block_size]
    rec = rec if values is not None else bf16_to_f64(rec)
    dn, dv = w.d_nope, w.d_v
    return rec[:, :dn], rec[:, dn: dn + dv], rec[:, dn + dv:]


def gqa_decode(gi: dict, batches=None, heads=None, values: np.ndarray | None = None):
    """Every query row (b, s, h) attends with [q_nope; q_rope] over its group's
    K = [K_nope ; k_rope] and V.  Returns dict(out [B, S_q, nh, d_v], lse [B, S_q, nh])."""
    w = gi["workload"]
    G = gi["groups"]
    batches = list(range(w.batch)) if batches is None else list(batches)
    heads = list(range(w.heads)) if heads is None else list(heads)
    q_nope = bf16_to_f64(gi["q_nope"])
    q_rope = bf16_to_f64(gi["q_rope"])
    out = np.zeros((len(batches), w.q_len, len(heads), w.d_v))
    lse = np.full((len(batches), w.q_len, len(heads)), -math.inf)
    for i, b in enumerate(batches):
        L = int(gi["seq_lens"][b])
        streams = {}
        for j, h in enumerate(heads):
            g = group_of(h, w.heads, G)
            if g not in streams:
                kn, v, kr = gqa_stream(gi, b, g, values)
                streams[g] = (np.concatenate([kn, kr], axis=1), v)
            k, v = streams[g]
            for s in range(w.q_len):
                q = np.concatenate([q_nope[b, s, h], q_rope[b, s, h]])
                _, out[i, s, j], lse[i, s, j] = attend(q, k, v, gi["softmax_scale"], visible_limit(L, w.q_len, s))
    return dict(out=out, lse=lse)
