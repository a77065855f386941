"""Benchmark: one absorbed-MLA decode step (absorb -> split-K paged decode ->
LSE merge fused with the up-projection) on one MI355X, on synthetic inputs.

Prints one JSON line.  ``value`` is the effective latent-cache read rate of
the whole step (algorithmic cache bytes / step time) with every input already
resident in HBM; the step time itself is ``ms_per_step`` (and ``us_per_step``),
timed over replays of HIP graphs that each run the steps of all input
replicas in order, as the attention of consecutive layers runs within one
captured forward pass (``--graph-steps 1``: one step per replay, also
reported as ``graph_1step_us_per_step``; ``--no-graph``: eager launches;
``--unfused``: separate merge and up-projection launches).  Per-call
times and the decode kernel's roofline come from an eager loop with HIP events
between the calls.
Consecutive steps rotate through independent replicas of all inputs whose
total exceeds three times the 256 MB Infinity Cache, so each step reads its
cache and weights from HBM.  With the headline workload the line also
carries the cache append, the prefill, the TPLA split, GQLA's two paths and
the decode step on every other decode workload (``configs``).

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload deepseek_v3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
INFINITY_CACHE_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, seq_lens):
    """Bytes and flops the method itself must move / compute for one step."""
    L = [int(x) for x in seq_lens]
    elem = 1 if w.cache_dtype == "fp8_e4m3" else 2
    rec = w.record_elems * elem + (4 if w.cache_dtype == "fp8_e4m3" else 0)
    cache_bytes = sum(L) * rec
    R = w.q_len * w.heads
    q_bytes = w.batch * R * (w.d_latent + w.d_rope) * 2          # q_lat + q_rope read by the decode
    w_bytes = 2 * w.heads * w.d_nope * w.d_latent * 2            # W_UK + W_UV
    io_bytes = w.batch * R * (w.d_nope + w.d_rope) * 2 + w.batch * R * w.d_v * (4 if w.out_dtype == "fp32" else 2)
    score_flops = pv_flops = 0
    for Lb in L:
        for s in range(w.q_len):
            vis = max(0, Lb - w.q_len + 1 + s)
            score_flops += 2 * w.heads * vis * (w.d_latent + w.d_rope)
            pv_flops += 2 * w.heads * vis * w.d_latent
    attn_flops = score_flops + pv_flops
    proj_flops = 4 * w.batch * R * w.d_nope * w.d_latent
    return dict(cache_bytes=cache_bytes, decode_bytes=cache_bytes + q_bytes,
                step_bytes=cache_bytes + w_bytes + io_bytes, attn_flops=attn_flops, score_flops=score_flops,
                pv_flops=pv_flops,
                step_flops=attn_flops + proj_flops, record_bytes=rec, tokens=sum(L))


KERNEL_SOURCES = ("decode.hip", "decode_wide.hip", "decode_wide_fp8.hip", "decode_wide_pair.hip", "wide_common.h",
                  "decode_common.h", "split_plan.h", "tile_ops.h", "mla_device.h", "mla_kernels.h")


def decode_kernel_name(w) -> str:
    if w.q_len * w.heads <= 64:
        return "decode_kernel"
    if w.cache_dtype == "fp8_e4m3":
        return "decode_f8_kernel"
    return "decode_wide_pair_kernel" if w.d_latent == 256 else "decode_wide_kernel"


def mfma_peak_tflops(w, alg) -> float:
    """The dense MFMA peak of the decode's products.  bf16 for a bf16 cache
    and for the few-rows kernel (which decodes e4m3 tiles to bf16).  The
    128-row e4m3 kernel runs the score product on e4m3 MFMA (5.0 PFLOP/s) and
    P . V on bf16 (2.5): its peak is the rate at which both finish at their
    own peaks, flops / (score / 5.0 + pv / 2.5)."""
    if w.cache_dtype != "fp8_e4m3" or w.q_len * w.heads <= 64:
        return MFMA_BF16_PEAK_TFLOPS
    t = alg["score_flops"] / MFMA_FP8_PEAK_TFLOPS + alg["pv_flops"] / MFMA_BF16_PEAK_TFLOPS
    return alg["attn_flops"] / t


def roofline_of(alg, us, measured=None, w=None):
    """The decode launch against the roofline that bounds it: HBM when its
    algorithmic flops per byte are below the ridge of the nominal peaks
    (the MFMA peak of its products over HBM), MFMA above it.  The other
    fraction is given beside it, and each against the measured peaks when
    there are any (the measured MFMA rate is bf16's)."""
    gbs = alg["decode_bytes"] / (us * 1e-6) / 1e9
    tflops = alg["attn_flops"] / (us * 1e-6) / 1e12
    ai = alg["attn_flops"] / alg["decode_bytes"]
    peak = MFMA_BF16_PEAK_TFLOPS if w is None else mfma_peak_tflops(w, alg)
    r = {"flop_per_byte": round(ai, 1)}
    if ai > peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        r.update(bound="mfma", achieved=round(tflops, 1), peak=round(peak, 1), unit="TFLOP/s",
                 frac=round(tflops / peak, 4), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
        if peak != MFMA_BF16_PEAK_TFLOPS:
            r["peak_is"] = "score product on e4m3 MFMA (5.0 PFLOP/s), P.V on bf16 (2.5), weighted by their flops"
            r["frac_of_bf16_peak"] = round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)
    else:
        r.update(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                 frac=round(gbs / HBM_PEAK_GBS, 4), mfma_frac=round(tflops / peak, 4))
    if measured:
        r["frac_of_measured_hbm"] = round(gbs / measured["hbm_gbs"], 4)
        r["frac_of_measured_mfma"] = round(tflops / measured["mfma_bf16_tflops"], 4)
    return r


def measured_peaks(torch, stream, reps: int = 5):
    """Reference points measured on this GPU with the library's calibration
    probes (HIP kernels, medians over reps, HIP events): the HBM read rate of
    mla_probe_hbm_read over 2 GiB (contiguous chunks per work-group,
    non-temporal 16-byte loads from every CU) and the bf16
    MFMA rate of mla_probe_mfma (independent 32x32x16 chains on every SIMD).
    Beside them, for context: a 1 GiB torch device copy (read + write bytes)
    and a bf16 GEMM of 8192^3 on the device's BLAS."""
    import numpy as np
    from head_latent_attention_absorbed_amd import mla_probe_hbm_read, mla_probe_mfma

    nbytes = 2 << 30
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    src = x[: x.numel() // 2]
    dst = torch.empty_like(src)
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda")
    iters = 20000
    flops = 0
    for _ in range(2):
        mla_probe_hbm_read(x, nbytes, sink, stream)
        flops = mla_probe_mfma(iters, sink, stream)
        dst.copy_(src)
        torch.matmul(a, b)
    torch.cuda.synchronize()
    t = {k: [] for k in ("read", "mfma", "copy", "mm")}
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        e[0].record(stream)
        mla_probe_hbm_read(x, nbytes, sink, stream)
        e[1].record(stream)
        mla_probe_mfma(iters, sink, stream)
        e[2].record(stream)
        dst.copy_(src)
        e[3].record(stream)
        torch.matmul(a, b)
        e[4].record(stream)
        torch.cuda.synchronize()
        for k, (i, j) in zip(t, ((0, 1), (1, 2), (2, 3), (3, 4))):
            t[k].append(e[i].elapsed_time(e[j]) * 1e-3)
    med = {k: float(np.median(v)) for k, v in t.items()}
    res = {"hbm_gbs": round(nbytes / med["read"] / 1e9, 1),
           "mfma_bf16_tflops": round(flops / med["mfma"] / 1e12, 1),
           "torch_copy_gbs": round(2 * src.numel() * 4 / med["copy"] / 1e9, 1),
           "blas_bf16_tflops": round(2 * 8192 ** 3 / med["mm"] / 1e12, 1),
           "how": "hbm_gbs: mla_probe_hbm_read over 2 GiB; mfma_bf16_tflops: mla_probe_mfma "
                  f"({iters} rounds); torch_copy_gbs: a 1 GiB fp32 device copy, read + write bytes; "
                  f"blas_bf16_tflops: torch.matmul bf16 8192^3; medians of {reps}"}
    del x, src, dst, a, b, sink
    torch.cuda.empty_cache()
    return res


def copy_pattern_gbs(torch, stream, st, alg, reps: int = 10):
    """The decode's own copy pattern alone (mla_probe_tile_copy: the same
    plan, grid and copy instructions over the same cache, no products):
    the launch's cache bytes over its median time, GB/s; None where the
    probe has no kernel (e4m3 cache, 64 query rows or fewer)."""
    import numpy as np
    from head_latent_attention_absorbed_amd import MlaError, mla_probe_tile_copy

    w = st.workload
    if w.cache_dtype != "bf16" or w.q_len * w.heads <= 64:
        return None
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    base = st.cache.data_ptr()
    args = (st.shape, base, base + w.d_latent * st.elem, st.token_stride, st.block_stride, st.block_table,
            st.seq_lens, st.num_parts, sink, stream)
    try:
        mla_probe_tile_copy(*args)
    except MlaError:
        return None
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        mla_probe_tile_copy(*args)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    return round(alg["cache_bytes"] / float(np.median(ts)) / 1e9, 1)


def host_info():
    """CPU model and the BLAS library numpy uses (for the CPU baseline)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = max(int(i.get("num_threads", 1)) for i in info)
    except Exception:
        pass
    return model, blas, threads


def kernel_source_hash() -> str:
    """sha256 over the sources the decode kernel is built from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "head_latent_attention_absorbed_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by a copy kernel's reading), or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_probe(mb: int, reps: int = 3):
    """A plain device copy of known size (read mb MB, write mb MB), launched
    after the timed region so that a counter run sees a kernel whose HBM bytes
    are known; its FETCH_SIZE / WRITE_SIZE readings calibrate the decode's."""
    import torch

    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} x add(out=) over {mb} MiB fp32 (read {n * 4} B, write {n * 4} B per launch)")


def cpu_baseline(inputs, budget_s: float):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload:
    whole sequences, all heads, until about ``budget_s`` seconds of CPU work.
    The timed region includes the oracle's decode of the whole paged cache to
    fp64 (its first step), not only the sampled sequences' attention."""
    import numpy as np
    import oracle

    w = inputs["workload"]
    t0 = time.perf_counter()
    values = oracle.cache_values(inputs)
    done, tokens = 0, 0
    while done < w.batch:
        oracle.decode_one(inputs, done, values=values)
        tokens += int(inputs["seq_lens"][done])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    elem = 1 if w.cache_dtype == "fp8_e4m3" else 2
    rec = w.record_elems * elem + (4 if w.cache_dtype == "fp8_e4m3" else 0)
    return dict(value=tokens * rec / dt / 1e12, unit="TB/s", seconds=dt, sequences=done, tokens=tokens)


def leg_prefill(torch, np, stream, K):
    """The MLA-form prefill of a prompt batch (keys and values expanded per
    head, then causal attention), each call timed with events."""
    from head_latent_attention_absorbed_amd import PrefillStep
    from workloads import make_prefill_inputs, prefill_workload
    pw, P = prefill_workload()
    pf = make_prefill_inputs(pw, P)
    pst = PrefillStep(pf)
    for _ in range(2):
        pst.run()
    torch.cuda.synchronize()
    KP = max(3, min(K, 10))
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(KP)]
    for i in range(KP):
        pev[i][0].record(stream)
        pst.kv()
        pev[i][1].record(stream)
        pst.attention()
        pev[i][2].record(stream)
    torch.cuda.synchronize()
    pkv_us = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in pev]))
    pat_us = float(np.median([e[1].elapsed_time(e[2]) * 1e3 for e in pev]))
    plens = [int(v) for v in pf["seq_lens"]]
    p_tokens = sum(plens)
    p_attn_flops = pw.heads * (pw.d_nope + pw.d_rope + pw.d_v) * 2 * sum(L * (L + 1) // 2 for L in plens)
    p_kv_flops = p_tokens * pw.heads * pw.d_latent * (pw.d_nope + pw.d_v) * 2
    return {
        "what": "mla_prefill_kv (K_nope, V per head from the records) + mla_prefill_attention (causal)",
        "workload": pw.name, "batch": pw.batch, "prompt_len": P, "seq_lens": plens, "heads": pw.heads,
        "tokens_per_s": round(p_tokens / ((pkv_us + pat_us) * 1e-6), 1),
        "kv_us_median": round(pkv_us, 2),
        "attention_us_median": round(pat_us, 2),
        "roofline": {"kernel": "prefill_kernel (mla_prefill_attention)", "bound": "mfma",
                     "achieved": round(p_attn_flops / (pat_us * 1e-6) / 1e12, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(p_attn_flops / (pat_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flops_per_launch": p_attn_flops},
        "kv_roofline": {"bound": "mfma", "achieved": round(p_kv_flops / (pkv_us * 1e-6) / 1e12, 1),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(p_kv_flops / (pkv_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                        "algorithmic_flops_per_call": p_kv_flops},
    }


def leg_tpla(torch, np, stream, K, args, w, inputs, alg, step0):
    """The TPLA latent split on one device: two Hadamard-basis shards of the
    measured decode (each over half the latent and the whole RoPE key),
    summed; each call timed with events, and the split's error against the
    MLA decode on the same inputs with and without the basis change."""
    from head_latent_attention_absorbed_amd import TplaStep, combine_up_supported, mla_tpla_rotate_cache
    if w.cache_dtype != "bf16" or not combine_up_supported(w.d_latent // 2, w.d_v):
        return None
    step0.run()
    torch.cuda.synchronize()
    mla_out = step0.out.float().clone()
    tp_err, tst, plain = {}, None, None
    for had in (False, True):
        t = TplaStep(inputs, 2, had, partial=args.partial)
        t.prepare()
        t.run()
        torch.cuda.synchronize()
        tp_err["hadamard" if had else "plain"] = float((t.out.float() - mla_out).norm() / mla_out.norm())
        if had:
            tst = t
        else:
            plain = t
    KT = max(3, min(K, 10))
    names = ("absorb", "decode", "combine_up")
    tev = [[torch.cuda.Event(enable_timing=True) for _ in range(3 * tst.n + 2)] for _ in range(KT)]
    for i in range(KT):
        e = tev[i]
        e[0].record(stream)
        for sh in range(tst.n):
            for j, nm in enumerate(names):
                getattr(tst, nm)(sh)
                e[1 + 3 * sh + j].record(stream)
        tst.reduce()
        e[-1].record(stream)
    torch.cuda.synchronize()
    tp_step = float(np.median([e[0].elapsed_time(e[-1]) * 1e3 for e in tev]))
    tp_dec = float(np.median([e[1 + 3 * sh].elapsed_time(e[2 + 3 * sh]) * 1e3 for e in tev for sh in range(tst.n)]))
    sh_bytes = alg["tokens"] * (tst.dcs + w.d_rope) * 2 + w.batch * w.q_len * w.heads * (tst.dcs + w.d_rope) * 2
    # the basis change of the whole cache (latent of every slot, read and written once)
    rev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    b0 = plain.base
    for i in range(3):
        rev[i].record(stream)
        mla_tpla_rotate_cache(b0.shape, b0.cache, b0.token_stride, b0.block_stride, plain.num_pages)
    rev[3].record(stream)
    torch.cuda.synchronize()
    rot_us = float(np.median([rev[i].elapsed_time(rev[i + 1]) * 1e3 for i in range(3)]))
    rot_bytes = 2 * plain.num_pages * w.block_size * w.d_latent * 2
    return {
        "what": "TPLA latent split on one GPU: 2 Hadamard-basis shards (absorb + decode + merge/up-proj "
                "at d_c/2 each) + mla_tpla_reduce",
        "n_shards": tst.n, "us_per_step": round(tp_step, 2), "shard_decode_us_median": round(tp_dec, 2),
        "rel_l2_vs_mla": {k: round(v, 5) for k, v in tp_err.items()},
        "roofline": {"kernel": "decode_wide_pair_kernel (one shard, d_latent %d)" % tst.dcs, "bound": "hbm",
                     "achieved": round(sh_bytes / (tp_dec * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(sh_bytes / (tp_dec * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": sh_bytes},
        "rotate_cache": {"us": round(rot_us, 2), "bytes": rot_bytes,
                         "achieved_gbs": round(rot_bytes / (rot_us * 1e-6) / 1e9, 1),
                         "frac": round(rot_bytes / (rot_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }


def leg_gqla(torch, np, stream, K, args):
    """GQLA's two decoding paths at s_q = 2 on a LLaMA-3-8B-shaped model
    (H = 32 in 8 groups, B = 16, context 8192): the absorbed MQA path over the
    latent and the GQA path over the per-group expanded cache, each call
    timed with events."""
    from head_latent_attention_absorbed_amd import DecodeStep, GqaStep
    from workloads import GQLA_GROUPS, get_workload, make_gqa_inputs, make_inputs
    gw = get_workload("gqla_gqa")
    g_in = make_inputs(gw)
    g_mla = DecodeStep(g_in, partial=args.partial)
    g_gqa = GqaStep(make_gqa_inputs(gw, GQLA_GROUPS), partial=args.partial)
    for _ in range(2):
        g_mla.run()
        g_gqa.run()
    torch.cuda.synchronize()
    KT = max(3, min(K, 10))
    paths = {"mqa_absorb": (g_mla, ("absorb", "decode", "combine_up")),
             "gqa": (g_gqa, ("queries", "decode", "combine", "output"))}
    g_res = {}
    for name, (st, calls) in paths.items():
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(KT)]
        for i in range(KT):
            ev[i][0].record(stream)
            for j, c in enumerate(calls):
                getattr(st, c)()
                ev[i][j + 1].record(stream)
        torch.cuda.synchronize()
        g_res[name] = {c: float(np.median([e[j].elapsed_time(e[j + 1]) * 1e3 for e in ev])) for j, c in
                       enumerate(calls)}
        g_res[name]["step"] = float(np.median([e[0].elapsed_time(e[-1]) * 1e3 for e in ev]))
    g_tokens = int(sum(int(x) for x in g_in["seq_lens"]))
    g_bytes = {"mqa_absorb": g_tokens * gw.record_elems * 2,
               "gqa": g_tokens * GQLA_GROUPS * (gw.d_nope + gw.d_v + gw.d_rope) * 2}
    # The GQA records repeat the shared RoPE key in every group (the record
    # layout used here; the method itself has one RoPE key per token): the
    # bytes with a single shared RoPE stream are given beside the measured
    # path's, so the comparison can be read without that inflation.
    rope_shared = g_tokens * (GQLA_GROUPS * (gw.d_nope + gw.d_v) + gw.d_rope) * 2
    return {
        "what": "GQLA's two decoding paths at s_q = 2, H = 32 in 8 groups, B = 16, context 8192: absorbed MQA "
                "over the latent vs GQA over per-group [K_nope | V | k_rope] records",
        "gqa_cache_bytes_with_one_rope_stream": rope_shared,
        "gqa_rope_repeat_factor": round(g_bytes["gqa"] / rope_shared, 4),
        "paths": {k: {"us_median": {c: round(t, 2) for c, t in v.items()}, "cache_bytes": g_bytes[k],
                      "decode_gbs": round(g_bytes[k] / (v["decode"] * 1e-6) / 1e9, 1),
                      "decode_frac": round(g_bytes[k] / (v["decode"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
                  for k, v in g_res.items()},
    }


DECODE_WORKLOADS = ("tiny", "deepseek_v3", "gqa7b", "tpla_shard", "kimi_k2_fp8")


def leg_configs(torch, np, stream, K, args, exclude, measured=None):
    """The decode step on every other decode workload, with HIP events
    between the calls of an eager loop (absorb, decode, merge with the
    up-projection).  Consecutive steps rotate through input replicas that
    together exceed three times the Infinity Cache where that takes at most
    16 replicas (``cold``); the 1.2 MB tiny workload cannot leave it, so its
    figures are warm."""
    from head_latent_attention_absorbed_amd import DecodeStep
    from workloads import get_workload, make_inputs

    res = {}
    for name in DECODE_WORKLOADS:
        if name == exclude:
            continue
        w = get_workload(name)
        inputs = make_inputs(w)
        alg = algorithmic(w, inputs["seq_lens"])
        need = math.ceil(3 * INFINITY_CACHE_BYTES / max(alg["step_bytes"], 1)) + 1
        nrep = min(16, max(3, need))
        steps = [DecodeStep(inputs, partial=args.partial) for _ in range(nrep)]
        for i in range(args.warmup):
            steps[i % nrep].run()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        for i in range(K):
            st, e = steps[i % nrep], ev[i]
            e[0].record(stream)
            st.absorb()
            e[1].record(stream)
            st.decode()
            e[2].record(stream)
            if st.fused:
                st.combine_up()
            else:
                st.combine()
                st.up()
            e[3].record(stream)
        torch.cuda.synchronize()
        t = np.array([[e[j].elapsed_time(e[j + 1]) * 1e3 for j in range(3)] for e in ev])
        step = t.sum(axis=1)
        dec_mean = float(t[:, 1].mean())
        med = np.median(t, axis=0)
        res[name] = {
            "batch": w.batch, "heads": w.heads, "q_len": w.q_len, "d_latent": w.d_latent, "cache": w.cache_dtype,
            "tokens": alg["tokens"], "cache_bytes": alg["cache_bytes"], "replicas": nrep, "cold": nrep >= need,
            "us_per_step": {"median": round(float(np.median(step)), 2),
                            "p10": round(float(np.percentile(step, 10)), 2),
                            "p90": round(float(np.percentile(step, 90)), 2)},
            "per_call_us_median": {"absorb": round(float(med[0]), 2), "decode": round(float(med[1]), 2),
                                   "merge_up": round(float(med[2]), 2)},
            "tbs_decode_merge": round(alg["cache_bytes"] / ((med[1] + med[2]) * 1e-6) / 1e12, 4),
            "tbs_step": round(alg["cache_bytes"] / (float(np.median(step)) * 1e-6) / 1e12, 4),
            "decode_roofline": dict(kernel=decode_kernel_name(w), **roofline_of(alg, dec_mean, measured, w)),
        }
        log(f"configs: {name} step {res[name]['us_per_step']['median']} us, decode {med[1]:.1f} us")
        del steps, inputs
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="deepseek_v3")
    ap.add_argument("--replicas", type=int, default=0, help="input replicas rotated across steps (0 = auto)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--partial", default="fp16", choices=("fp16", "fp32"), help="element type of the split partials")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run a plain copy of this many MiB (counter calibration)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step as eager launches instead of one HIP-graph replay")
    ap.add_argument("--graph-steps", type=int, default=0,
                    help="steps per graph replay (consecutive replicas, like the layers of one forward "
                         "pass); 0 = all replicas, 1 = one step per replay")
    ap.add_argument("--legs", dest="legs", action="store_true", default=None,
                    help="also time the prefill, TPLA-split and GQLA legs and the other decode workloads "
                         "(default: with the headline workload)")
    ap.add_argument("--decode-only", dest="legs", action="store_false", help="time the decode step only")
    ap.add_argument("--no-configs", action="store_true",
                    help="with the legs, leave out the decode step on the other decode workloads")
    ap.add_argument("--unfused", action="store_true",
                    help="merge (mla_combine_lse) and up-project (mla_up_v) in two launches")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; run with --gpus 1 "
                                   "(no multi-GPU path exists: sharding is described, not built)"}))
        sys.exit(2)

    import numpy as np
    import torch

    from head_latent_attention_absorbed_amd import DecodeStep
    from workloads import get_workload, make_inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    w = get_workload(args.workload)
    t0 = time.perf_counter()
    inputs = make_inputs(w)
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s")
    alg = algorithmic(w, inputs["seq_lens"])
    per_rep = alg["step_bytes"]
    nrep = args.replicas or max(3, math.ceil(3 * INFINITY_CACHE_BYTES / max(per_rep, 1)) + 1)
    nrep = min(nrep, 64)
    steps = [DecodeStep(inputs, partial=args.partial, fused=False if args.unfused else None) for _ in range(nrep)]
    calls = ("absorb", "decode", "combine_up_v") if steps[0].fused else ("absorb", "decode", "combine", "up_v")
    stream = torch.cuda.current_stream()
    log(f"workload {w.name}: tokens={alg['tokens']} cache={alg['cache_bytes'] / 1e6:.1f} MB "
        f"replicas={nrep} num_parts={steps[0].num_parts}")

    for i in range(args.warmup):
        steps[i % nrep].run()
    torch.cuda.synchronize()

    K = args.steps
    # Whole-step time: each replica's step captured once as a HIP graph (its
    # kernels, no host work between them) and replayed; --no-graph times
    # the eager loop below instead.
    graph_ms = None
    graph1_ms = None
    warm_ms = None
    R = nrep if args.graph_steps <= 0 else min(args.graph_steps, nrep)
    if not args.no_graph:
        from head_latent_attention_absorbed_amd import capture_steps

        for st in steps:
            st.capture()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        # One step per replay (each replica's own graph).
        for i in range(args.warmup):
            steps[i % nrep].replay()
        torch.cuda.synchronize()
        g0.record(stream)
        for i in range(K):
            steps[(args.warmup + i) % nrep].replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph1_ms = g0.elapsed_time(g1) / K
        # Warm: one replica's graph over and over (its cache stays in the
        # Infinity Cache when it fits; the headline cache does not, 236 MB).
        g0.record(stream)
        for i in range(K):
            steps[0].replay()
        g1.record(stream)
        torch.cuda.synchronize()
        warm_ms = g0.elapsed_time(g1) / K
        # R consecutive replicas per replay, as the layers of one forward pass:
        # K // R such replays plus K % R single-step ones, K steps in all.
        graph_ms = graph1_ms
        if R > 1:
            multi = capture_steps(steps[:R])
            for i in range(max(1, args.warmup // R)):
                multi.replay()
            torch.cuda.synchronize()
            g0.record(stream)
            for i in range(K // R):
                multi.replay()
            for i in range(K % R):
                steps[i].replay()
            g1.record(stream)
            torch.cuda.synchronize()
            graph_ms = g0.elapsed_time(g1) / K

    # Per-call times: the same steps as eager launches with HIP events
    # between the calls, on the stream the kernels run on.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        st = steps[(args.warmup + i) % nrep]
        e = ev[i]
        e[0].record(stream)
        st.absorb()
        e[1].record(stream)
        st.decode()
        e[2].record(stream)
        if st.fused:
            st.combine_up()
            e[3].record(stream)
        else:
            st.combine()
            e[3].record(stream)
            st.up()
            e[4].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    eager_ms = total_ms / K
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    per_call = {name: [ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in range(K)]
                for j, name in enumerate(calls)}
    med = {k: float(np.median(v)) for k, v in per_call.items()}
    eager_steps = np.sum([per_call[c] for c in calls], axis=0)
    dec_us = float(np.mean(per_call["decode"]))

    # The cache append (x . [W_DKV | W_KR] -> RoPE -> records in the pages),
    # timed on its own over the same replicas: events around each call.
    from workloads import make_append_inputs
    ap = make_append_inputs(w)
    for st in steps:
        st.set_append_inputs(ap)
    for i in range(3):
        steps[i % nrep].append()
    torch.cuda.synchronize()
    aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        aev[i][0].record(stream)
        steps[(args.warmup + i) % nrep].append()
        aev[i][1].record(stream)
    torch.cuda.synchronize()
    app_us = [a.elapsed_time(b) * 1e3 for a, b in aev]
    app_med = float(np.median(app_us))
    M = w.batch * w.q_len
    app_bytes = w.d_model * (w.d_latent + w.d_rope) * 2 + M * w.d_model * 2 + M * alg["record_bytes"]

    run_legs = args.legs if args.legs is not None else (args.workload == "deepseek_v3")
    prefill_res = leg_prefill(torch, np, stream, K) if run_legs else None
    tpla_res = leg_tpla(torch, np, stream, K, args, w, inputs, alg, steps[0]) if run_legs else None
    gqla_res = leg_gqla(torch, np, stream, K, args) if run_legs else None
    measured = measured_peaks(torch, stream) if run_legs else None
    copy_gbs = copy_pattern_gbs(torch, stream, steps[0], alg)
    configs_res = (leg_configs(torch, np, stream, K, args, w.name, measured)
                   if run_legs and not args.no_configs else None)

    us_step = ms_per_step * 1e3
    value = alg["cache_bytes"] / (us_step * 1e-6) / 1e12
    result = {
        "metric": "decode-attn us/step + effective latent-cache TB/s, B=32 H=128 ctx 8K",
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(us_step, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3+bf16" if w.cache_dtype == "fp8_e4m3" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.batch, "heads": w.heads, "q_len": w.q_len, "d_latent": w.d_latent, "d_rope": w.d_rope,
            "d_nope": w.d_nope, "d_v": w.d_v, "block_size": w.block_size, "cache": w.cache_dtype,
            "seq_lens": f"uniform[{w.seq_len[0]},{w.seq_len[1]}] seed {w.seed}",
            "tokens": alg["tokens"], "cache_bytes": alg["cache_bytes"], "input_replicas": nrep,
            "num_parts": steps[0].num_parts, "partials": args.partial,
            "merge": "fused with up-projection" if steps[0].fused else "separate launches",
        },
        "step_launch": (f"hip_graph, {R} steps (replicas) per replay" if R > 1 else "hip_graph, 1 step per replay")
                       if graph_ms is not None else "eager",
        "graph_1step_us_per_step": round(graph1_ms * 1e3, 2) if graph1_ms is not None else None,
        "eager_us_per_step": round(eager_ms * 1e3, 2),
        "eager_step_us": {"median": round(float(np.median(eager_steps)), 2),
                          "p10": round(float(np.percentile(eager_steps, 10)), 2),
                          "p90": round(float(np.percentile(eager_steps, 90)), 2)},
        "warm_graph_1step_us_per_step": round(warm_ms * 1e3, 2) if warm_ms is not None else None,
        "per_call_us_median": {k: round(v, 2) for k, v in med.items()},
        "tbs_decode_merge": round(alg["cache_bytes"] / (sum(med[c] for c in calls[1:]) * 1e-6) / 1e12, 4),
        "step_hbm_frac": round(value * 1e3 / HBM_PEAK_GBS, 4),
        "roofline": dict(
            kernel=f"{decode_kernel_name(w)} (mla_decode_paged)",
            **roofline_of(alg, dec_us, measured, w),
            traffic=measured_traffic(w.name, decode_kernel_name(w)) if args.partial == "fp16" else None,
            algorithmic_bytes_per_launch=alg["decode_bytes"],
            algorithmic_flops_per_launch=alg["attn_flops"],
            avg_launch_us=round(dec_us, 2),
            copy_pattern_gbs=copy_gbs,
            frac_of_copy_pattern=(round(alg["decode_bytes"] / (dec_us * 1e-6) / 1e9 / copy_gbs, 4)
                                  if copy_gbs else None),
        ),
        "measured_peaks": measured,
        "wall_s": round(wall, 3),
        "append": {
            "what": "mla_append_kv: new tokens' [c_KV | k_rope] records from x [B*S_q, d_model] "
                    "(product, RoPE, paged write)",
            "d_model": w.d_model,
            "us_median": round(app_med, 2),
            "roofline": {"bound": "hbm", "achieved": round(app_bytes / (app_med * 1e-6) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(app_bytes / (app_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_call": app_bytes},
        },
        "tpla": tpla_res,
        "gqla": gqla_res,
        "prefill": prefill_res,
        "configs": configs_res,
    }
    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(inputs, args.cpu_budget)
        model, blas, threads = host_info()
        result["cpu_baseline"] = {
            "value": round(cb["value"], 8), "unit": "TB/s", "cores": threads, "kind": "oracle",
            "sample": f"{cb['sequences']} of {w.batch} sequences ({cb['tokens']} tokens, all {w.heads} heads) "
                      f"in {cb['seconds']:.1f}s (with the fp64 decode of the whole cache), numpy fp64 "
                      f"explicit K/V reconstruction",
            "cpu": model, "blas": blas,
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
