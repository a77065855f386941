"""The seeded input generator: reproducibility, encodings and the paged layout."""
import numpy as np
import torch

from workloads import WORKLOADS, Workload, make_inputs, f32_to_bf16_bits, f32_to_e4m3_bits, small_workload


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 50000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38], dtype=np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_e4m3_encoding_is_nearest_even():
    from oracle import e4m3_to_f64
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(20000) * 60).astype(np.float32)
    codes = f32_to_e4m3_bits(x)
    table = e4m3_to_f64(np.arange(256, dtype=np.uint8))
    finite = np.where(np.isnan(table), np.inf, table)
    xc = np.clip(x.astype(np.float64), -448, 448)
    best = np.min(np.abs(finite[None, :] - xc[:, None]), axis=1)
    got = np.abs(e4m3_to_f64(codes) - xc)
    assert np.all(got <= best + 1e-300)


def test_reproducible_and_seed_sensitive():
    w = small_workload("deepseek_v3", batch=3, seq_len=(70, 200), max_seq_len=256)
    a, b = make_inputs(w), make_inputs(w)
    for k in ("q_nope", "q_rope", "w_uk", "w_uv", "cache", "block_table", "seq_lens"):
        assert np.array_equal(a[k], b[k]), k
    c = make_inputs(w, seed=w.seed + 1)
    assert not np.array_equal(a["q_nope"], c["q_nope"])


def test_paged_layout_and_poison():
    w = small_workload("deepseek_v3", batch=4, seq_len=(1, 300), max_seq_len=320, spare_blocks=3,
                       forced_lens=(0, 64, 65))
    inp = make_inputs(w)
    L = inp["seq_lens"]
    assert list(L[:3]) == [0, 64, 65]
    bt = inp["block_table"]
    nblk = [(-(-int(x) // 64)) for x in L]
    used = np.concatenate([bt[b, : nblk[b]] for b in range(w.batch)])
    assert len(set(used.tolist())) == len(used) == sum(nblk)           # distinct pages
    assert used.min() >= 0 and used.max() < inp["num_blocks"]
    for b in range(w.batch):
        assert np.all(bt[b, nblk[b]:] == -1)                           # unused entries poisoned
        if L[b] % 64:
            tail = inp["cache"][bt[b, nblk[b] - 1], L[b] % 64:]
            assert np.all(tail == 0x7FC0)                               # slots past the length are NaN
    # the permutation really permutes
    assert not np.array_equal(np.sort(used), used)


def test_fp8_scale_rule():
    w = small_workload("kimi_k2_fp8", batch=2, seq_len=(5, 70), max_seq_len=128)
    inp = make_inputs(w)
    from oracle import e4m3_to_f64
    bt, L = inp["block_table"], inp["seq_lens"]
    for b in range(w.batch):
        t = np.arange(L[b])
        codes = inp["cache"][bt[b, t // 64], t % 64]
        scale = inp["kv_scale"][bt[b, t // 64], t % 64]
        assert np.all(np.isfinite(scale)) and np.all(scale > 0)
        mags = np.max(np.abs(e4m3_to_f64(codes)), axis=1)
        assert np.all(mags <= 448) and np.all(mags >= 416)   # amax maps to (nearly) 448


def test_named_workloads_match_the_configs():
    d = WORKLOADS
    assert (d["tiny"].batch, d["tiny"].heads, d["tiny"].seq_len, d["tiny"].paged) == (1, 16, (1024, 1024), False)
    assert (d["deepseek_v3"].batch, d["deepseek_v3"].heads, d["deepseek_v3"].seq_len) == (32, 128, (4096, 8192))
    assert (d["gqa7b"].batch, d["gqa7b"].heads, d["gqa7b"].seq_len) == (16, 32, (8192, 8192))
    t = d["tpla_shard"]
    assert (t.batch, t.heads, t.d_latent, t.seq_len, t.out_dtype, t.weight_var) == (8, 128, 256, (32768, 32768), "fp32", 1 / 256)
    k = d["kimi_k2_fp8"]
    assert (k.batch, k.heads, k.q_len, k.seq_len, k.cache_dtype) == (16, 64, 4, (16384, 32768), "fp8_e4m3")
    g = d["gqla_gqa"]
    assert (g.batch, g.heads, g.q_len, g.seq_len, g.d_nope, g.d_v) == (16, 32, 2, (8192, 8192), 128, 128)
    for w in d.values():
        assert abs(w.softmax_scale - 192 ** -0.5) < 1e-15
        assert w.seed == 1000 + ("tiny", "deepseek_v3", "gqa7b", "tpla_shard", "kimi_k2_fp8", "gqla_gqa").index(w.name)


def test_gqa_inputs_layout():
    """Per-group streams: own pages, the shared RoPE key repeated in every
    group's record, poison past the length, reproducible."""
    from workloads import make_gqa_inputs

    w = small_workload("gqla_gqa", batch=3, seq_len=(5, 130), max_seq_len=192, forced_lens=(130, 1, 0), spare_blocks=2)
    a, b = make_gqa_inputs(w, 4), make_gqa_inputs(w, 4)
    assert all(np.array_equal(a[k], b[k]) for k in ("q_nope", "cache", "block_table"))
    G, bs = 4, w.block_size
    pages = a["block_table"][a["block_table"] >= 0]
    assert len(pages) == len(set(pages.tolist()))                     # no page shared by two streams
    assert np.array_equal(a["stream_lens"], np.repeat(a["seq_lens"], G))
    dn, dv = w.d_nope, w.d_v
    for bq in range(3):
        L = int(a["seq_lens"][bq])
        t = np.arange(L)
        recs = [a["cache"][a["block_table"][bq * G + g, t // bs], t % bs] for g in range(G)]
        for g in range(1, G):
            assert np.array_equal(recs[g][:, dn + dv:], recs[0][:, dn + dv:])        # one RoPE key per token
            assert L == 0 or not np.array_equal(recs[g][:, :dn], recs[0][:, :dn])    # own K_nope per group
        if L % bs:
            last = a["block_table"][bq * G, (L - 1) // bs]
            assert np.all(a["cache"][last, L % bs:] == 0x7FC0)                       # poisoned tail
