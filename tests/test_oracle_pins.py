"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each pin is a ``check_*`` function taking the oracle module, so that
``test_planted_mistakes_are_caught`` can hand it a copy with a deliberate bug
and show that the pin fails.
"""
import math
import os
import types
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import oracle.mla_oracle as om
from workloads import Workload, make_inputs, f32_to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))
BF16_ONE = np.uint16(0x3F80)


def tiny(**kw) -> Workload:
    base = dict(name="tiny_pin", batch=2, heads=3, q_len=1, d_latent=16, seq_len=(5, 11), paged=True,
                cache_dtype="bf16", out_dtype="bf16", weight_var=1.0 / 16, seed=7, d_nope=8, d_rope=4,
                d_v=8, block_size=4, spare_blocks=2)
    base.update(kw)
    return Workload(**base)


def close(a, b, tol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs err {err:.3e} > {tol:.1e} x {scale:.3g}"


def f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


# ------------------------------------------------------------------ P1 absorb identity

def check_absorb_identity(o):
    """Scores through the absorbed query equal scores against explicitly
    reconstructed keys (the absorb of W_UK into the query is exact)."""
    inp = make_inputs(tiny(q_len=2))
    w = inp["workload"]
    qn, qr, wk, wv = f64(inp["q_nope"]), f64(inp["q_rope"]), f64(inp["w_uk"]), f64(inp["w_uv"])
    q_lat = o.absorb_q(qn, wk)
    for b in range(w.batch):
        C, KR = o.gather(inp, b)
        for h in range(w.heads):
            k, _ = o.reconstruct_kv(C, KR, wk[h:h + 1], wv[h:h + 1])
            for s in range(w.q_len):
                explicit = w.softmax_scale * (k[0] @ np.concatenate([qn[b, s, h], qr[b, s, h]]))
                absorbed = o.absorbed_scores(q_lat[b, s, h], qr[b, s, h], C, KR, w.softmax_scale)
                close(absorbed, explicit)


def test_p1_absorb_identity():
    check_absorb_identity(oracle)


# ------------------------------------------------------------------ P2 softmax sums to 1

def check_softmax_sums_to_one(o):
    rng = np.random.default_rng(3)
    for L in (1, 2, 17, 300):
        k = rng.standard_normal((L, 12)) * 3
        v = rng.standard_normal((L, 5))
        q = rng.standard_normal(12)
        for limit in (L, max(1, L // 2)):
            p, _, _ = o.attend(q, k, v, 0.3, limit)
            assert p.shape == (limit,)
            assert abs(float(np.sum(p)) - 1.0) <= 1e-12
            assert np.all(p >= 0)


def test_p2_softmax_sums_to_one():
    check_softmax_sums_to_one(oracle)


# ------------------------------------------------------------------ P3 one token

def check_single_token(o):
    """With one cached token the output is that token's value and lse its score."""
    inp = make_inputs(tiny(seq_len=(1, 1)))
    w = inp["workload"]
    qn, qr, wk, wv = f64(inp["q_nope"]), f64(inp["q_rope"]), f64(inp["w_uk"]), f64(inp["w_uv"])
    res = o.decode(inp)
    for b in range(w.batch):
        page = inp["block_table"][b, 0]
        rec = f64(inp["cache"][page, 0])
        c, kr = rec[: w.d_latent], rec[w.d_latent:]
        for h in range(w.heads):
            v0 = np.array([sum(c[i] * wv[h, i, j] for i in range(w.d_latent)) for j in range(w.d_v)])
            k0 = np.concatenate([[sum(wk[h, n, i] * c[i] for i in range(w.d_latent)) for n in range(w.d_nope)], kr])
            z0 = w.softmax_scale * float(np.dot(k0, np.concatenate([qn[b, 0, h], qr[b, 0, h]])))
            close(res["out"][b, 0, h], v0)
            close([res["lse"][b, 0, h]], [z0])
            close(res["o_lat"][b, 0, h], c)


def test_p3_single_token():
    check_single_token(oracle)


# ------------------------------------------------------------------ P4 paged == contiguous

def check_paged_equals_contiguous(o):
    wp = tiny(paged=True, seq_len=(3, 13), q_len=2)
    wc = replace(wp, paged=False)
    a, b = make_inputs(wp), make_inputs(wc)
    assert not np.array_equal(a["block_table"], b["block_table"])
    ra, rb = o.decode(a), o.decode(b)
    for key in ("out", "lse", "o_lat"):
        assert np.array_equal(ra[key], rb[key]), key


def test_p4_paged_equals_contiguous():
    check_paged_equals_contiguous(oracle)


# ------------------------------------------------------------------ P5 zero query

def check_zero_query_mean(o):
    """q = 0 gives uniform weights, so the output is the mean value over visible tokens."""
    inp = make_inputs(tiny(q_len=3, seq_len=(4, 9)))
    inp["q_nope"][:] = 0
    inp["q_rope"][:] = 0
    w = inp["workload"]
    wv = f64(inp["w_uv"])
    res = o.decode(inp)
    for b in range(w.batch):
        L = int(inp["seq_lens"][b])
        t = np.arange(L)
        recs = f64(inp["cache"][inp["block_table"][b, t // w.block_size], t % w.block_size])
        for s in range(w.q_len):
            n = L - w.q_len + 1 + s
            for h in range(w.heads):
                mean_v = (recs[:n, : w.d_latent] @ wv[h]).mean(axis=0)
                close(res["out"][b, s, h], mean_v)
                close([res["lse"][b, s, h]], [math.log(n)])


def test_p5_zero_query_mean():
    check_zero_query_mean(oracle)


# ------------------------------------------------------------------ P6 GQA special case

def check_gqa_special_case(o):
    """GQA written as MLA: the latent holds the keys and values of g groups, W_UK[h]
    and W_UV[h] select head h's group and the RoPE parts are zero.  The result must be
    grouped-query attention, computed here by torch's SDPA in fp64."""
    dn, g, H, S = 4, 2, 4, 2
    w = tiny(heads=H, q_len=S, d_nope=dn, d_v=dn, d_latent=2 * g * dn, d_rope=2, seq_len=(3, 10),
             weight_var=1.0)
    inp = make_inputs(w)
    inp["q_rope"][:] = 0
    inp["cache"][..., w.d_latent:] = 0
    wk = np.zeros((H, dn, w.d_latent), dtype=np.uint16)
    wv = np.zeros((H, w.d_latent, dn), dtype=np.uint16)
    grp = [h * g // H for h in range(H)]
    for h in range(H):
        for n in range(dn):
            wk[h, n, grp[h] * dn + n] = BF16_ONE
            wv[h, g * dn + grp[h] * dn + n, n] = BF16_ONE
    inp["w_uk"], inp["w_uv"] = wk, wv
    res = o.decode(inp)
    qn = f64(inp["q_nope"])
    for b in range(w.batch):
        L = int(inp["seq_lens"][b])
        t = np.arange(L)
        recs = f64(inp["cache"][inp["block_table"][b, t // w.block_size], t % w.block_size])
        keys = recs[:, : g * dn].reshape(L, g, dn).transpose(1, 0, 2)        # [g, L, dn]
        vals = recs[:, g * dn: 2 * g * dn].reshape(L, g, dn).transpose(1, 0, 2)
        q = torch.from_numpy(qn[b].transpose(1, 0, 2).copy())                  # [H, S, dn]
        kk = torch.from_numpy(keys).repeat_interleave(H // g, dim=0)
        vv = torch.from_numpy(vals).repeat_interleave(H // g, dim=0)
        mask = torch.tensor([[t_ <= L - S + s for t_ in range(L)] for s in range(S)])
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, scale=w.softmax_scale)
        close(res["out"][b], ref.numpy().transpose(1, 0, 2))


def test_p6_gqa_special_case():
    check_gqa_special_case(oracle)


# ------------------------------------------------------------------ P7 SDPA cross-check

def check_sdpa_crosscheck(o):
    """Random weights, several query tokens: keys/values rebuilt with torch and
    attended by torch's SDPA (explicit scale and boolean causal mask)."""
    w = tiny(q_len=3, seq_len=(3, 14), heads=4)
    inp = make_inputs(w)
    res = o.decode(inp)
    qn, qr, wk, wv = (torch.from_numpy(f64(inp[k])) for k in ("q_nope", "q_rope", "w_uk", "w_uv"))
    for b in range(w.batch):
        L = int(inp["seq_lens"][b])
        t = np.arange(L)
        recs = torch.from_numpy(f64(inp["cache"][inp["block_table"][b, t // w.block_size], t % w.block_size]))
        c, kr = recs[:, : w.d_latent], recs[:, w.d_latent:]
        k_nope = torch.einsum("hnc,tc->htn", wk, c)
        k = torch.cat([k_nope, kr.unsqueeze(0).expand(w.heads, L, w.d_rope)], dim=2)
        v = torch.einsum("tc,hcv->htv", c, wv)
        q = torch.cat([qn[b], qr[b]], dim=2).permute(1, 0, 2)
        mask = torch.zeros(w.q_len, L, dtype=torch.bool)
        for s in range(w.q_len):
            mask[s, : L - w.q_len + 1 + s] = True
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.softmax_scale)
        close(res["out"][b], ref.permute(1, 0, 2).numpy())


def test_p7_sdpa_crosscheck():
    check_sdpa_crosscheck(oracle)


# ------------------------------------------------------------------ P8 split + merge

def check_split_merge(o):
    """Merging the oracle's partials over any partition of the positions by their
    log-sum-exp reproduces the unsplit result (online softmax is exact)."""
    w = tiny(q_len=2, seq_len=(6, 23))
    inp = make_inputs(w)
    res = o.decode(inp)
    rng = np.random.default_rng(11)
    for b in range(w.batch):
        L = int(inp["seq_lens"][b])
        for _ in range(3):
            cuts = sorted(set(rng.integers(0, L + 1, size=3).tolist()) | {0, L})
            parts = [o.partial(inp, b, a, c) for a, c in zip(cuts[:-1], cuts[1:])]
            o_m, lse_m = o.combine(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            close(o_m, res["o_lat"][b])
            close(lse_m, res["lse"][b])
    # an empty split (past every visible position) weighs nothing
    o_e, lse_e = o.partial(inp, 0, int(inp["seq_lens"][0]), int(inp["seq_lens"][0]) + 5)
    assert np.all(o_e == 0) and np.all(np.isneginf(lse_e))
    o_all, lse_all = o.combine(np.stack([o_e, o_e]), np.stack([lse_e, lse_e]))
    assert np.all(o_all == 0) and np.all(np.isneginf(lse_all))


def test_p8_split_merge():
    check_split_merge(oracle)


# ------------------------------------------------------------------ P9 up-projection

def check_up_projection(o):
    """sum_t p_t (c_t W_UV) = (sum_t p_t c_t) W_UV: the latent output through W_UV
    equals the explicitly reconstructed-V output."""
    inp = make_inputs(tiny(q_len=2))
    res = o.decode(inp)
    close(o.up_v(res["o_lat"], f64(inp["w_uv"])), res["out"])


def test_p9_up_projection():
    check_up_projection(oracle)


# ------------------------------------------------------------------ P10 order invariance

def check_order_invariance(o):
    """With one query token every cached position is visible, so shuffling the
    records among the sequence's slots leaves the result unchanged."""
    w = tiny(seq_len=(7, 15))
    inp = make_inputs(w)
    ref = o.decode(inp)
    rng = np.random.default_rng(5)
    flat = inp["cache"].reshape(-1, w.record_elems)
    for b in range(w.batch):
        L = int(inp["seq_lens"][b])
        t = np.arange(L)
        idx = inp["block_table"][b, t // w.block_size].astype(np.int64) * w.block_size + t % w.block_size
        flat[idx] = flat[idx[rng.permutation(L)]]
    got = o.decode(inp)
    close(got["out"], ref["out"])
    close(got["lse"], ref["lse"])


def test_p10_order_invariance():
    check_order_invariance(oracle)


# ------------------------------------------------------------------ P11 brute force

def check_brute_force(o):
    """Pure-Python scalar loops (no numpy arithmetic) on a tiny case."""
    w = Workload(name="bf", batch=1, heads=2, q_len=2, d_latent=8, seq_len=(5, 5), paged=True,
                 cache_dtype="bf16", out_dtype="bf16", weight_var=0.25, seed=99, d_nope=4, d_rope=2,
                 d_v=4, block_size=2, spare_blocks=1)
    inp = make_inputs(w)
    res = o.decode(inp)
    bt = inp["block_table"].tolist()
    cache = f64(inp["cache"]).tolist()
    qn, qr = f64(inp["q_nope"]).tolist(), f64(inp["q_rope"]).tolist()
    wk, wv = f64(inp["w_uk"]).tolist(), f64(inp["w_uv"]).tolist()
    L = int(inp["seq_lens"][0])
    scale = 1.0 / math.sqrt(w.d_nope + w.d_rope)
    for h in range(w.heads):
        for s in range(w.q_len):
            zs, vs = [], []
            for t in range(L - w.q_len + 1 + s):
                rec = cache[bt[0][t // w.block_size]][t % w.block_size]
                c, kr = rec[: w.d_latent], rec[w.d_latent:]
                key = [sum(wk[h][n][i] * c[i] for i in range(w.d_latent)) for n in range(w.d_nope)] + kr
                val = [sum(c[i] * wv[h][i][j] for i in range(w.d_latent)) for j in range(w.d_v)]
                qv = qn[0][s][h] + qr[0][s][h]
                zs.append(scale * sum(a * b for a, b in zip(qv, key)))
                vs.append(val)
            m = max(zs)
            es = [math.exp(z - m) for z in zs]
            tot = sum(es)
            out = [sum(es[i] * vs[i][j] for i in range(len(es))) / tot for j in range(w.d_v)]
            close(res["out"][0, s, h], out)
            close([res["lse"][0, s, h]], [m + math.log(tot)])


def test_p11_brute_force():
    check_brute_force(oracle)


# ------------------------------------------------------------------ P12 / P13 decoders

def check_e4m3_decoder(o):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = o.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert got[0x7E] == 448.0


def test_p12_e4m3_decoder():
    check_e4m3_decoder(oracle)


def check_bf16_decoder(o):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    exp_all_ones = (bits & 0x7F80) == 0x7F80
    bits = bits[~exp_all_ones]
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(o.bf16_to_f64(bits), ref)


def test_p13_bf16_decoder():
    check_bf16_decoder(oracle)


# ------------------------------------------------------------------ P14 causal tail

def check_causal_tail(o):
    """Query s of an S_q-token step at length L equals a one-token step at
    length L - S_q + 1 + s with the same cache."""
    w = tiny(q_len=3, seq_len=(4, 12))
    inp = make_inputs(w)
    res = o.decode(inp)
    for s in range(w.q_len):
        one = dict(inp)
        one["workload"] = replace(w, q_len=1)
        one["q_nope"] = inp["q_nope"][:, s: s + 1].copy()
        one["q_rope"] = inp["q_rope"][:, s: s + 1].copy()
        one["seq_lens"] = (inp["seq_lens"] - w.q_len + 1 + s).astype(np.int32)
        r1 = o.decode(one)
        close(r1["out"][:, 0], res["out"][:, s])
        close(r1["lse"][:, 0], res["lse"][:, s])


def test_p14_causal_tail():
    check_causal_tail(oracle)


# ------------------------------------------------------------------ idle batch slot

def test_idle_slot_reads_nothing():
    """A sequence of length 0 sees no position: output 0 and lse -inf, and the
    other sequences of the batch are unaffected."""
    w = tiny(batch=3, forced_lens=(0, 7, 0), q_len=2, seq_len=(5, 9))
    inp = make_inputs(w)
    res = oracle.decode(inp)
    for b in (0, 2):
        assert np.all(res["out"][b] == 0) and np.all(np.isneginf(res["lse"][b]))
    one = oracle.decode(inp, batches=[1])
    assert np.array_equal(one["out"][0], res["out"][1])


# ------------------------------------------------------------------ P15 record size

def test_p15_record_size_against_printed_figures():
    from workloads import WORKLOADS
    rows = {}
    with open(os.path.join(HERE, "golden", "record_size.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, val, per_tok, _ = [x.strip() for x in line.split("|", 3)]
                rows[name] = (float(val), int(per_tok))
    rec = WORKLOADS["deepseek_v3"].record_elems
    assert rec == 576
    val, n = rows["kv_kept_llama2_7b"]
    assert round(100.0 * rec / n, 2) == val
    val, n = rows["kv_cut_llama2_7b"]
    assert round(100.0 * (1 - rec / n), 2) == val
    val, n = rows["kv_kept_llama3_8b"]
    assert 100.0 * rec / n == val
    for name in ("tiny", "deepseek_v3", "gqa7b", "kimi_k2_fp8"):
        assert WORKLOADS[name].record_elems == 576


def check_prefill_sdpa(m):
    """MLA-form prefill against torch's causal scaled-dot-product attention
    on keys and values rebuilt here with torch from the raw weights."""
    from workloads import make_prefill_inputs
    w = tiny(batch=2, heads=3, seq_len=(9, 9), forced_lens=(9, 6))
    pf = make_prefill_inputs(w, prompt_len=9)
    res = m.prefill(pf)
    t = lambda bits: torch.from_numpy(m.bf16_to_f64(bits))
    w_uk, w_uv = t(pf["w_uk"]), t(pf["w_uv"])
    for b in range(w.batch):
        L = int(pf["seq_lens"][b])
        rec = t(pf["ckr"][b, :L])
        c, kr = rec[:, :w.d_latent], rec[:, w.d_latent:]
        k = torch.cat([torch.einsum("hnc,tc->htn", w_uk, c), kr.expand(w.heads, L, w.d_rope)], dim=2)
        v = torch.einsum("tc,hcv->htv", c, w_uv)
        q = torch.cat([t(pf["q_nope"][b, :L]), t(pf["q_rope"][b, :L])], dim=2).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=pf["softmax_scale"])
        close(res["out"][b, :L], ref.permute(1, 0, 2).numpy(), 1e-10)
        assert np.all(np.isnan(res["out"][b, L:]))


def test_p16_prefill_sdpa():
    check_prefill_sdpa(oracle)


# ------------------------------------------------------------------ P17-P19 e4m3 cache with per-token scale
#
# The e4m3 cache stores each token's record as OCP E4M3 codes plus one fp32
# scale, and a cached value is code x scale (FP8 KV quantization named in the
# TransMLA abstracts; one scale per token over the whole record is this
# build's reading).  These pins fix how the scale enters, independently of
# the oracle's own e4m3 branch.

def _fp8_tiny(**kw):
    base = dict(cache_dtype="fp8_e4m3", q_len=2, seq_len=(5, 14), heads=3)
    base.update(kw)
    return tiny(**base)


def _e4m3_torch(codes):
    """e4m3 bytes -> fp64 through torch's float8_e4m3fn (a library decoder)."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def _valid_slots(inp):
    """(page, slot) of every cached position of every sequence."""
    w = inp["workload"]
    out = []
    for b in range(w.batch):
        for t in range(int(inp["seq_lens"][b])):
            out.append((int(inp["block_table"][b, t // w.block_size]), t % w.block_size))
    return out


def check_e4m3_pow2_scales_equal_bf16_cache(o):
    """Give every token a power-of-two scale 2^k (k != 0 for most tokens):
    every e4m3 value times 2^k is then exactly a bf16 value, so decoding the
    e4m3 cache must give, bit for bit, what decoding a bf16 cache holding
    those products gives.  Dividing by the scale, dropping it, or taking it
    from the wrong (page, slot) breaks the equality."""
    inp = make_inputs(_fp8_tiny())
    w = inp["workload"]
    rng = np.random.default_rng(23)
    kv_scale = inp["kv_scale"].copy()
    bf = np.full(inp["cache"].shape, 0x7FC0, dtype=np.uint16)          # NaN where nothing is cached
    for page, slot in _valid_slots(inp):
        k = int(rng.choice([-5, -3, -2, -1, 1, 2, 3, 4]))
        kv_scale[page, slot] = np.float32(2.0 ** k)
        vals = _e4m3_torch(inp["cache"][page, slot]) * 2.0 ** k          # exact in fp64
        bits = f32_to_bf16_bits(vals.astype(np.float32))
        assert np.array_equal(f64(bits), vals), "e4m3 x 2^k must be a bf16 value"
        bf[page, slot] = bits
    inp["kv_scale"] = kv_scale
    ref_inp = dict(inp)
    ref_inp["workload"] = replace(w, cache_dtype="bf16")
    ref_inp["cache"] = bf
    ref_inp["kv_scale"] = None
    got, ref = o.decode(inp), o.decode(ref_inp)
    for key in ("out", "lse", "o_lat"):
        assert np.array_equal(got[key], ref[key]), key


def test_p17_e4m3_pow2_scales_equal_bf16_cache():
    check_e4m3_pow2_scales_equal_bf16_cache(oracle)


def check_e4m3_sdpa(o):
    """The generated scales (amax / 448): keys and values rebuilt with torch
    from the codes (torch's e4m3 decoder) times kv_scale[page][slot], attended
    by torch's SDPA in fp64 with the causal tail as a mask."""
    w = _fp8_tiny(q_len=3, heads=4, seq_len=(3, 15))
    inp = make_inputs(w)
    res = o.decode(inp)
    qn, qr, wk, wv = (torch.from_numpy(f64(inp[k])) for k in ("q_nope", "q_rope", "w_uk", "w_uv"))
    for b in range(w.batch):
        L = int(inp["seq_lens"][b])
        t = np.arange(L)
        pages, slots = inp["block_table"][b, t // w.block_size], t % w.block_size
        recs = torch.from_numpy(_e4m3_torch(inp["cache"][pages, slots]))
        recs = recs * torch.from_numpy(inp["kv_scale"][pages, slots].astype(np.float64)).unsqueeze(1)
        c, kr = recs[:, : w.d_latent], recs[:, w.d_latent:]
        k = torch.cat([torch.einsum("hnc,tc->htn", wk, c), kr.unsqueeze(0).expand(w.heads, L, w.d_rope)], dim=2)
        v = torch.einsum("tc,hcv->htv", c, wv)
        q = torch.cat([qn[b], qr[b]], dim=2).permute(1, 0, 2)
        mask = torch.zeros(w.q_len, L, dtype=torch.bool)
        for s in range(w.q_len):
            mask[s, : L - w.q_len + 1 + s] = True
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.softmax_scale)
        close(res["out"][b], ref.permute(1, 0, 2).numpy())


def test_p18_e4m3_sdpa():
    check_e4m3_sdpa(oracle)


def check_e4m3_brute_force(o):
    """Pure-Python scalar loops over an e4m3 record: each code is looked up in
    torch's table of the 256 e4m3 values, times the token's scale as a Python
    float; keys, values, softmax and output in scalar arithmetic."""
    w = Workload(name="bf8", batch=1, heads=2, q_len=2, d_latent=8, seq_len=(6, 6), paged=True,
                 cache_dtype="fp8_e4m3", out_dtype="bf16", weight_var=0.25, seed=98, d_nope=4, d_rope=2,
                 d_v=4, block_size=2, spare_blocks=1)
    inp = make_inputs(w)
    res = o.decode(inp)
    table = _e4m3_torch(np.arange(256, dtype=np.uint8)).tolist()
    bt = inp["block_table"].tolist()
    codes, scales = inp["cache"].tolist(), inp["kv_scale"].tolist()
    qn, qr = f64(inp["q_nope"]).tolist(), f64(inp["q_rope"]).tolist()
    wk, wv = f64(inp["w_uk"]).tolist(), f64(inp["w_uv"]).tolist()
    L = int(inp["seq_lens"][0])
    scale = 1.0 / math.sqrt(w.d_nope + w.d_rope)
    for h in range(w.heads):
        for s in range(w.q_len):
            zs, vs = [], []
            for t in range(L - w.q_len + 1 + s):
                page, slot = bt[0][t // w.block_size], t % w.block_size
                rec = [table[x] * scales[page][slot] for x in codes[page][slot]]
                c, kr = rec[: w.d_latent], rec[w.d_latent:]
                key = [sum(wk[h][n][i] * c[i] for i in range(w.d_latent)) for n in range(w.d_nope)] + kr
                val = [sum(c[i] * wv[h][i][j] for i in range(w.d_latent)) for j in range(w.d_v)]
                qv = qn[0][s][h] + qr[0][s][h]
                zs.append(scale * sum(a * b for a, b in zip(qv, key)))
                vs.append(val)
            m = max(zs)
            es = [math.exp(z - m) for z in zs]
            tot = sum(es)
            out = [sum(es[i] * vs[i][j] for i in range(len(es))) / tot for j in range(w.d_v)]
            close(res["out"][0, s, h], out)
            close([res["lse"][0, s, h]], [m + math.log(tot)])


def test_p19_e4m3_brute_force():
    check_e4m3_brute_force(oracle)


# ------------------------------------------------------------------ planted mistakes

def _mutant(**patches):
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update({k: getattr(om, k) for k in dir(om) if not k.startswith("__")})
    # Re-bind the functions so that their global lookups see the patches.
    for name in dir(om):
        fn = getattr(om, name)
        if isinstance(fn, types.FunctionType) and fn.__module__ == om.__name__:
            m.__dict__[name] = types.FunctionType(fn.__code__, m.__dict__, name, fn.__defaults__, fn.__closure__)
    m.__dict__.update(patches)
    return m


def _no_rope_kv(C, KR, w_uk, w_uv):
    k, v = om.reconstruct_kv(C, KR, w_uk, w_uv)
    k = k.copy()
    k[:, :, w_uk.shape[1]:] = 0
    return k, v


def _w_uv_transposed(o_lat, w_uv):
    return np.einsum("...hc,hvc->...hv", o_lat, w_uv.reshape(w_uv.shape[0], w_uv.shape[2], w_uv.shape[1]))


def _off_by_one_limit(L, q_len, s):
    return max(0, L - q_len + s)


def _e4m3_bias8(bits):
    return om.e4m3_to_f64(bits) * 0.5


def _bad_combine(o_parts, lse_parts):
    lse_parts = np.asarray(lse_parts)
    m = np.max(lse_parts, axis=0)
    wts = np.exp(lse_parts - m)
    return np.einsum("k...,k...d->...d", wts, o_parts), m  # forgets to normalise


def _e4m3_values(inputs):
    return om.e4m3_to_f64(inputs["cache"])


def _cache_values_scale_dropped(inputs):
    if inputs["workload"].cache_dtype == "bf16":
        return om.bf16_to_f64(inputs["cache"])
    return _e4m3_values(inputs)


def _cache_values_scale_divided(inputs):
    if inputs["workload"].cache_dtype == "bf16":
        return om.bf16_to_f64(inputs["cache"])
    return _e4m3_values(inputs) / inputs["kv_scale"].astype(np.float64)[..., None]


def _cache_values_scale_slot_major(inputs):
    """The scale array read as [slot][page] instead of [page][slot]."""
    if inputs["workload"].cache_dtype == "bf16":
        return om.bf16_to_f64(inputs["cache"])
    ks = inputs["kv_scale"]
    wrong = ks.reshape(-1).reshape(ks.shape[1], ks.shape[0]).T
    return _e4m3_values(inputs) * wrong.astype(np.float64)[..., None]


def _cache_values_scale_per_page(inputs):
    """One scale per page (its first slot's) broadcast over the page."""
    if inputs["workload"].cache_dtype == "bf16":
        return om.bf16_to_f64(inputs["cache"])
    return _e4m3_values(inputs) * inputs["kv_scale"].astype(np.float64)[:, :1, None]


def _sign_flip_absorb(q_nope, w_uk):
    return -om.absorb_q(q_nope, w_uk)


@pytest.mark.parametrize("patch,check", [
    (dict(reconstruct_kv=_no_rope_kv), check_sdpa_crosscheck),
    (dict(reconstruct_kv=_no_rope_kv), check_brute_force),
    (dict(visible_limit=_off_by_one_limit), check_sdpa_crosscheck),
    (dict(visible_limit=_off_by_one_limit), check_zero_query_mean),
    (dict(up_v=_w_uv_transposed), check_up_projection),
    (dict(e4m3_to_f64=_e4m3_bias8), check_e4m3_decoder),
    (dict(combine=_bad_combine), check_split_merge),
    (dict(absorb_q=_sign_flip_absorb), check_absorb_identity),
    (dict(reconstruct_kv=_no_rope_kv), check_prefill_sdpa),
    (dict(cache_values=_cache_values_scale_dropped), check_e4m3_pow2_scales_equal_bf16_cache),
    (dict(cache_values=_cache_values_scale_divided), check_e4m3_pow2_scales_equal_bf16_cache),
    (dict(cache_values=_cache_values_scale_slot_major), check_e4m3_pow2_scales_equal_bf16_cache),
    (dict(cache_values=_cache_values_scale_per_page), check_e4m3_pow2_scales_equal_bf16_cache),
    (dict(cache_values=_cache_values_scale_dropped), check_e4m3_sdpa),
    (dict(cache_values=_cache_values_scale_divided), check_e4m3_sdpa),
    (dict(cache_values=_cache_values_scale_slot_major), check_e4m3_sdpa),
    (dict(cache_values=_cache_values_scale_per_page), check_e4m3_sdpa),
    (dict(cache_values=_cache_values_scale_dropped), check_e4m3_brute_force),
    (dict(cache_values=_cache_values_scale_divided), check_e4m3_brute_force),
    (dict(cache_values=_cache_values_scale_slot_major), check_e4m3_brute_force),
    (dict(e4m3_to_f64=_e4m3_bias8), check_e4m3_sdpa),
])
def test_planted_mistakes_are_caught(patch, check):
    with pytest.raises(AssertionError):
        check(_mutant(**patch))
