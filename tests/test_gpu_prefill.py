"""Parity of the MLA-form prefill (mla_prefill_kv + mla_prefill_attention,
through the C ABI) with the fp64 oracle: reconstructed keys and values, and
causal attention at every position of ragged, padded prompts."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from workloads import make_prefill_inputs, prefill_workload, small_workload
from gpu_helpers import compare, to_np, tolerances

pytestmark = pytest.mark.gpu

CASES = {
    # (workload, prompt_len): ragged prompts, a tile tail, lengths 1 and 0
    "h8_p300": (small_workload("deepseek_v3", batch=3, heads=8, seq_len=(1, 300), forced_lens=(300, 131, 1)), 300),
    "h8_idle": (small_workload("deepseek_v3", batch=2, heads=8, seq_len=(1, 97), forced_lens=(0, 97)), 97),
    "dc256_h16": (small_workload("tpla_shard", batch=2, heads=16, seq_len=(33, 160), forced_lens=(160, 33)), 160),
    "h128_p96": (small_workload("deepseek_v3", batch=1, heads=128, seq_len=(96, 96)), 96),
    # a prompt shorter than one key tile, and single-position prompts
    "h8_p20": (small_workload("deepseek_v3", batch=3, heads=8, seq_len=(1, 20), forced_lens=(20, 1, 13)), 20),
}


def prefill_tolerances(w):
    """The decode's bounds (rel L2 5e-3, twice for e4m3) with max |err| 2e-2:
    the prefill stores the reconstructed keys and values in bf16 before the
    attention, and an early position averages a few value rows of size up to
    ~4, whose bf16 rounding alone reaches 4 * 2^-9 = 0.008 before the output's
    own rounding."""
    tol_abs, tol_rel = tolerances(w)
    return 2 * tol_abs, tol_rel


def _model_with_bf16_kv(pf, b, heads, positions):
    """The oracle's attention over keys and values rounded to bf16, the
    precision the prefill stores them in.  What remains between this model
    and the kernel is the bf16 rounding of the probabilities fed to the
    value product and of the output: at most 2^-9 (|o| + 2 max|V|), about
    1e-2 for the few-token averages of the first positions (max|V| ~ 4)."""
    w = pf["workload"]
    L = int(pf["seq_lens"][b])
    rec = oracle.bf16_to_f64(pf["ckr"][b, :L])
    K, V = oracle.reconstruct_kv(rec[:, :w.d_latent], rec[:, w.d_latent:], oracle.bf16_to_f64(pf["w_uk"])[heads],
                                 oracle.bf16_to_f64(pf["w_uv"])[heads])
    K = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(K))
    V = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(V))
    qn = oracle.bf16_to_f64(pf["q_nope"][b])
    qr = oracle.bf16_to_f64(pf["q_rope"][b])
    out = np.zeros((len(positions), len(heads), w.d_v))
    for i, s in enumerate(positions):
        for j, h in enumerate(heads):
            q = np.concatenate([qn[s, h], qr[s, h]])
            out[i, j] = oracle.attend(q, K[j], V[j], pf["softmax_scale"], s + 1)[1]
    return out


def untile_kv(x, B, H, P):
    """[B, 32 T, H, 128] view of a tile-native key or value buffer: tile j of
    (b, h) is 16 granule rows g of 32 slots, position 32 j + t in slot
    t ^ (4 (g & 1))."""
    T = (P + 31) // 32
    x = np.asarray(x).reshape(B, H, T, 16, 32, 8)
    g = np.arange(16)[:, None]
    t = np.arange(32)[None, :]
    y = x[:, :, :, g, t ^ (4 * (g & 1)), :]            # [B, H, T, 16 (g), 32 (t), 8]
    return y.transpose(0, 2, 4, 1, 3, 5).reshape(B, T * 32, H, 128)


def _run(pf):
    import torch
    from head_latent_attention_absorbed_amd import PrefillStep

    st = PrefillStep(pf)
    for t in (st.k_nope, st.v, st.out, st.lse):
        t.fill_(float("nan"))
    st.run()
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_parity(name):
    w, P = CASES[name]
    pf = make_prefill_inputs(w, P)
    print(f"[case] prefill {name}: B={w.batch} H={w.heads} P={P} d_c={w.d_latent} lens={list(pf['seq_lens'])}",
          flush=True)
    st = _run(pf)
    tol_abs, tol_rel = tolerances(w)
    # keys and values of every position < L_b (bf16 results of fp32 sums);
    # the rest of the last tile is zero
    k_got = untile_kv(to_np(st.k_nope), w.batch, w.heads, P)
    v_got = untile_kv(to_np(st.v), w.batch, w.heads, P)
    for b in range(w.batch):
        L = int(pf["seq_lens"][b])
        if L == 0:
            continue
        rec = oracle.bf16_to_f64(pf["ckr"][b, :L])
        K, V = oracle.reconstruct_kv(rec[:, :w.d_latent], rec[:, w.d_latent:], oracle.bf16_to_f64(pf["w_uk"]),
                                     oracle.bf16_to_f64(pf["w_uv"]))
        compare(f"k_nope[{b}]", k_got[b, :L].transpose(1, 0, 2), K[:, :, :w.d_nope], tol_abs, tol_rel)
        compare(f"v[{b}]", v_got[b, :L].transpose(1, 0, 2), V, tol_abs, tol_rel)
        end = -(-L // 32) * 32
        assert np.all(k_got[b, L:end] == 0) and np.all(v_got[b, L:end] == 0), "tail of the last tile not zero"
    ref = oracle.prefill(pf)
    out, lse = to_np(st.out), to_np(st.lse)
    p_abs, p_rel = prefill_tolerances(w)
    for b in range(w.batch):
        L = int(pf["seq_lens"][b])
        compare(f"out[{b}]", out[b, :L], ref["out"][b, :L], p_abs, p_rel)
        compare(f"lse[{b}]", lse[b, :L], ref["lse"][b, :L], p_abs, p_rel)
        assert np.all(np.isnan(out[b, L:])) and np.all(np.isnan(lse[b, L:])), "wrote past the prompt"
        if L:
            pos = sorted({min(s, L - 1) for s in (0, 1, 31, 32, L // 2, L - 1)})
            heads = [0, w.heads - 1]
            model = _model_with_bf16_kv(pf, b, heads, pos)
            compare(f"out[{b}] vs bf16-K/V model", out[b][pos][:, heads], model, 1e-2, 2.5e-3)


def test_prefill_headline_sampled():
    """The prompt batch the prefill is measured on (DeepSeek-V3 heads, two
    prompts padded to 4096 positions): sampled positions (first, tile
    edges, the shorter prompt's last, the end) of sampled heads against the
    oracle; every computed output finite, padding untouched."""
    w, P = prefill_workload()
    pf = make_prefill_inputs(w, P)
    print(f"[case] prefill headline-sampled P={P} lens={list(pf['seq_lens'])}", flush=True)
    st = _run(pf)
    heads = [0, 77, 127]
    L1 = int(pf["seq_lens"][1])
    positions = sorted({0, 31, 32, 127, 128, 1023, 2047, L1 - 1, P - 1})
    ref = oracle.prefill(pf, heads=heads, positions=positions)
    out, lse = to_np(st.out), to_np(st.lse)
    p_abs, p_rel = prefill_tolerances(w)
    for b in range(w.batch):
        L = int(pf["seq_lens"][b])
        ps = [s for s in positions if s < L]
        compare(f"out[{b}] sampled", out[b][ps][:, heads], ref["out"][b][ps][:, heads], p_abs, p_rel)
        compare(f"lse[{b}] sampled", lse[b][ps][:, heads], ref["lse"][b][ps][:, heads], p_abs, p_rel)
        assert np.all(np.isfinite(out[b, :L])) and np.all(np.isfinite(lse[b, :L]))
        assert np.all(np.isnan(out[b, L:])), "wrote past the prompt"
