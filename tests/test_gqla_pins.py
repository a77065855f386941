"""Pins of the GQLA GQA-path oracle against what the mathematics fixes:

* torch's scaled-dot-product attention over keys and values repeated for
  the heads of each group (consecutive heads share a group), with the causal
  tail of a two-token step as an explicit mask;
* the two decoding paths of one set of GQLA weights agree: with the heads of
  a group sharing W_UK / W_UV, GQA attention over the group's expanded keys
  and values equals the absorbed MLA decode over the latent (the MLA oracle);
* planted mistakes (interleaved head groups, keys without the RoPE part)
  break the first pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.gqla_oracle as gq
from workloads import make_gqa_inputs, make_inputs, small_workload


def _gi(groups=4, **kw):
    w = small_workload("gqla_gqa", batch=3, heads=8, seq_len=(3, 70), max_seq_len=128, forced_lens=(70, 2, 0), **kw)
    return make_gqa_inputs(w, groups)


def _sdpa(gi):
    """Reference with torch: per head, its group's K = [K_nope; k_rope], V."""
    w = gi["workload"]
    G, H, S = gi["groups"], w.heads, w.q_len
    hpg = H // G
    out = np.zeros((w.batch, S, H, w.d_v))
    t = lambda a: torch.from_numpy(oracle.bf16_to_f64(a))
    for b in range(w.batch):
        L = int(gi["seq_lens"][b])
        if L == 0:
            continue
        ks, vs = [], []
        for g in range(G):
            pages = gi["block_table"][b * G + g, np.arange(L) // w.block_size]
            rec = t(gi["cache"][pages, np.arange(L) % w.block_size])
            ks.append(torch.cat([rec[:, : w.d_nope], rec[:, w.d_nope + w.d_v:]], dim=1))
            vs.append(rec[:, w.d_nope: w.d_nope + w.d_v])
        k = torch.stack(ks).repeat_interleave(hpg, dim=0)            # [H, L, d_n + d_r]
        v = torch.stack(vs).repeat_interleave(hpg, dim=0)
        q = torch.cat([t(gi["q_nope"][b]), t(gi["q_rope"][b])], dim=2).permute(1, 0, 2)  # [H, S, .]
        mask = torch.arange(L)[None, :] <= (L - S + torch.arange(S))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=gi["softmax_scale"])
        out[b] = ref.permute(1, 0, 2).numpy()
    return out


def _check_sdpa(m, gi):
    got = m.gqa_decode(gi)["out"]
    ref = _sdpa(gi)
    live = gi["seq_lens"] > 0
    return np.allclose(got[live], ref[live], rtol=0, atol=1e-10)


@pytest.mark.parametrize("groups", [1, 2, 4, 8])
def test_gqa_against_torch_sdpa(groups):
    gi = _gi(groups)
    assert _check_sdpa(gq, gi)
    assert np.all(gq.gqa_decode(gi)["out"][2] == 0)                    # idle sequence


def test_two_paths_of_one_weight_set_agree():
    """GQLA: heads of a group share W_UK / W_UV.  Expand the latent cache per
    group in fp64 and run the GQA path; it must equal the absorbed MLA decode."""
    G = 4
    w = small_workload("gqla_gqa", batch=2, heads=8, seq_len=(3, 70), max_seq_len=128, forced_lens=(70, 9))
    inp = make_inputs(w)
    hpg = w.heads // G
    # group-shared weights: heads of a group take their group's first head's matrices
    share = np.repeat(np.arange(0, w.heads, hpg), hpg)
    inp = dict(inp, w_uk=inp["w_uk"][share], w_uv=inp["w_uv"][share])
    mla = oracle.decode(inp)
    # the per-group expanded cache, fp64, streams laid out page after page
    MB, bs = w.max_blocks_per_seq, w.block_size
    rec = w.d_nope + w.d_v + w.d_rope
    values = np.full((w.batch * G * MB, bs, rec), np.nan)
    table = np.arange(w.batch * G * MB, dtype=np.int32).reshape(w.batch * G, MB)
    w_uk, w_uv = oracle.bf16_to_f64(inp["w_uk"]), oracle.bf16_to_f64(inp["w_uv"])
    for b in range(w.batch):
        C, KR = oracle.gather(inp, b)
        L = C.shape[0]
        heads = [g * hpg for g in range(G)]
        K, V = oracle.reconstruct_kv(C, KR, w_uk[heads], w_uv[heads])
        t = np.arange(L)
        for g in range(G):
            values[table[b * G + g, t // bs], t % bs] = np.concatenate([K[g][:, : w.d_nope], V[g], KR], axis=1)
    gi = dict(workload=w, groups=G, q_nope=inp["q_nope"], q_rope=inp["q_rope"], seq_lens=inp["seq_lens"],
              block_table=table, cache=None, softmax_scale=inp["softmax_scale"])
    gqa = gq.gqa_decode(gi, values=values)
    assert np.allclose(gqa["out"], mla["out"], rtol=0, atol=1e-10)
    assert np.allclose(gqa["lse"], mla["lse"], rtol=0, atol=1e-10)


def test_planted_interleaved_groups_fail(monkeypatch):
    monkeypatch.setattr(gq, "group_of", lambda h, heads, groups: h % groups)
    assert not _check_sdpa(gq, _gi(4))


def test_planted_keys_without_rope_fail(monkeypatch):
    real = gq.gqa_stream

    def no_rope(gi, b, g, values=None):
        kn, v, kr = real(gi, b, g, values)
        return kn, v, np.zeros_like(kr)

    monkeypatch.setattr(gq, "gqa_stream", no_rope)
    assert not _check_sdpa(gq, _gi(4))
