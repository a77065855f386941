"""One decode step on device: the C-ABI calls in order on one stream.

``DecodeStep`` holds device copies of a workload's inputs (torch tensors used
as plain device buffers), allocates the intermediate and output buffers, and
issues mla_absorb_q -> mla_decode_paged -> mla_combine_up_v (the merge and
the up-projection in one launch), or with ``fused=False`` the separate
mla_combine_lse -> mla_up_v, which also writes the merged latent rows o_lat.
"""
from __future__ import annotations

import numpy as np

from .binding import (
    MLA_BF16, MLA_FP8_E4M3, MLA_FP16, MLA_FP32, MLA_TILE_TOKENS, MlaShape,
    mla_absorb_q, mla_append_kv, mla_append_kv_noalloc, mla_append_kv_workspace_bytes, mla_decode_num_parts, mla_decode_paged,
    mla_combine_lse, mla_combine_up_v, mla_prefill_attention, mla_prefill_kv, mla_prefill_kv_elems,
    mla_prefill_workspace_bytes, mla_tpla_reduce, mla_tpla_rotate_cache, mla_tpla_split_weights, mla_up_v,
    mla_gqa_output, mla_gqa_queries,
)


def combine_up_supported(d_latent: int, d_v: int) -> bool:
    """Shapes mla_combine_up_v has a kernel for (it returns MLA_ERR_UNSUPPORTED otherwise)."""
    return d_latent in (256, 512) and d_v in (64, 128)


def split_plan(seq_lens, num_parts: int, tile: int = MLA_TILE_TOKENS):
    """The documented split plan of mla_decode_paged: a list of
    (slot, sequence, first position, end position) for every partial written.
    W is the fewest tiles per part for which the sequences' parts,
    ceil(n_b / W) each, fit in num_parts slots; sequence b's parts take
    consecutive slots in sequence order."""
    lens = [int(x) for x in seq_lens]
    if num_parts < len(lens):
        raise ValueError("num_parts must be at least the batch size")
    n = [(L + tile - 1) // tile if L > 0 else 0 for L in lens]
    if sum(n) == 0:
        return []
    W = 1
    while sum((x + W - 1) // W for x in n) > num_parts:
        W += 1
    plan, slot = [], 0
    for b, nb in enumerate(n):
        for j in range((nb + W - 1) // W):
            t0, t1 = j * W, min((j + 1) * W, nb)
            plan.append((slot, b, t0 * tile, min(t1 * tile, lens[b])))
            slot += 1
    return plan


def _dev_bits(torch, arr: np.ndarray, device, dtype):
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(dtype)
    return torch.from_numpy(a).to(device)


class DecodeStep:
    def __init__(self, inputs: dict, device: str = "cuda", num_parts: int | None = None, partial: str = "fp16",
                 fused: bool | None = None):
        """``partial`` is the element type of the split partials o_part:
        "fp16" (half the bytes) or "fp32".  ``fused``: merge and up-project in
        one launch (default where a kernel exists); o_lat is then None."""
        import torch

        if partial not in ("fp16", "fp32"):
            raise ValueError(f"partial must be 'fp16' or 'fp32', not {partial!r}")
        self.torch = torch
        w = inputs["workload"]
        self.workload = w
        fp8 = w.cache_dtype == "fp8_e4m3"
        self.shape = MlaShape.make(
            batch=w.batch, num_heads=w.heads, q_len=w.q_len, d_latent=w.d_latent, d_nope=w.d_nope,
            d_rope=w.d_rope, d_v=w.d_v, block_size=w.block_size, max_blocks_per_seq=w.max_blocks_per_seq,
            softmax_scale=float(inputs["softmax_scale"]), cache_dtype=MLA_FP8_E4M3 if fp8 else MLA_BF16,
            out_dtype=MLA_FP32 if w.out_dtype == "fp32" else MLA_BF16,
            partial_dtype=MLA_FP16 if partial == "fp16" else MLA_FP32)
        bf16 = torch.bfloat16
        self.q_nope = _dev_bits(torch, inputs["q_nope"], device, bf16)
        self.q_rope = _dev_bits(torch, inputs["q_rope"], device, bf16)
        self.w_uk = _dev_bits(torch, inputs["w_uk"], device, bf16)
        self.w_uv = _dev_bits(torch, inputs["w_uv"], device, bf16)
        self.cache = _dev_bits(torch, inputs["cache"], device, bf16)
        self.kv_scale = None if inputs["kv_scale"] is None else torch.from_numpy(inputs["kv_scale"]).to(device)
        self.block_table = torch.from_numpy(inputs["block_table"]).to(device)
        self.seq_lens = torch.from_numpy(inputs["seq_lens"]).to(device)
        self.elem = 1 if fp8 else 2
        self.token_stride = w.record_elems * self.elem
        self.block_stride = w.block_size * self.token_stride
        self.num_parts = num_parts if num_parts is not None else mla_decode_num_parts(self.shape)
        B, S, H, DC = w.batch, w.q_len, w.heads, w.d_latent
        R = S * H
        f32 = torch.float32
        self.q_lat = torch.empty((B, S, H, DC), dtype=bf16, device=device)
        self.o_part = torch.empty((self.num_parts, R, DC), dtype=torch.float16 if partial == "fp16" else f32,
                                  device=device)
        self.lse_part = torch.empty((self.num_parts, R), dtype=f32, device=device)
        supported = combine_up_supported(DC, w.d_v)
        if fused and not supported:
            raise ValueError(f"no fused merge + up-projection kernel for d_latent {DC}, d_v {w.d_v}")
        self.fused = supported if fused is None else bool(fused)
        self.o_lat = None if self.fused else torch.empty((B, S, H, DC), dtype=f32, device=device)
        self.lse = torch.empty((B, S, H), dtype=f32, device=device)
        self.out = torch.empty((B, S, H, w.d_v), dtype=f32 if w.out_dtype == "fp32" else bf16, device=device)

    def set_append_inputs(self, ap: dict):
        """Device copies of the cache-append inputs (hidden states x and the
        combined [W_DKV | W_KR]) and the append's workspace."""
        torch = self.torch
        device = self.q_nope.device
        self.x = _dev_bits(torch, ap["x"], device, torch.bfloat16)
        self.w_dkv = _dev_bits(torch, ap["w_dkv"], device, torch.bfloat16)
        self.rope_base = float(ap["rope_base"])
        self.d_model = int(ap["x"].shape[-1])
        nbytes = mla_append_kv_workspace_bytes(self.shape, self.d_model)
        self.append_ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)

    def append(self, stream=None, cache=None, kv_scale=None, noalloc=False):
        """Write the new tokens' records [c_KV | k_rope] into the cache;
        ``noalloc`` uses mla_append_kv_noalloc (the library's fixed scratch
        instead of this step's workspace)."""
        cache = self.cache if cache is None else cache
        kv_scale = self.kv_scale if kv_scale is None else kv_scale
        base = cache.data_ptr()
        if noalloc:
            mla_append_kv_noalloc(self.shape, self.d_model, self.x, self.w_dkv, self.rope_base, base,
                                  base + self.workload.d_latent * self.elem, self.token_stride, self.block_stride,
                                  kv_scale, self.block_table, self.seq_lens, stream)
            return
        mla_append_kv(self.shape, self.d_model, self.x, self.w_dkv, self.rope_base, base,
                      base + self.workload.d_latent * self.elem, self.token_stride, self.block_stride, kv_scale,
                      self.block_table, self.seq_lens, self.append_ws, self.append_ws.numel(), stream)

    def absorb(self, stream=None):
        mla_absorb_q(self.shape, self.q_nope, self.w_uk, self.q_lat, stream)

    def decode(self, stream=None, cache=None, kv_scale=None):
        cache = self.cache if cache is None else cache
        kv_scale = self.kv_scale if kv_scale is None else kv_scale
        base = cache.data_ptr()
        mla_decode_paged(self.shape, self.q_lat, self.q_rope, base, base + self.workload.d_latent * self.elem,
                         self.token_stride, self.block_stride, kv_scale, self.block_table, self.seq_lens,
                         self.num_parts, self.o_part, self.lse_part, stream)

    def combine(self, stream=None):
        mla_combine_lse(self.shape, self.num_parts, self.o_part, self.lse_part, self.seq_lens, self.o_lat, self.lse,
                        stream)

    def up(self, stream=None):
        mla_up_v(self.shape, self.o_lat, self.w_uv, self.out, stream)

    def combine_up(self, stream=None):
        mla_combine_up_v(self.shape, self.num_parts, self.o_part, self.lse_part, self.seq_lens, self.w_uv, self.out,
                         self.lse, stream)

    def finish(self, stream=None):
        """Merge of the splits and up-projection: one launch when fused, else two."""
        if self.fused:
            self.combine_up(stream)
        else:
            self.combine(stream)
            self.up(stream)

    def run(self, stream=None, cache=None, kv_scale=None):
        """The whole step: absorb, split-K decode, LSE merge, up-projection."""
        self.absorb(stream)
        self.decode(stream, cache, kv_scale)
        self.finish(stream)
        return self.out

    def capture(self):
        """Record the whole step (its launches, no allocation, no host
        work) into a HIP graph; replay() then issues it with one launch.  The
        graph reads and writes this step's buffers in place, so new inputs are
        copied into them (q_nope, q_rope, cache, seq_lens, block_table ...)
        before a replay.  The library's one-time kernel attribute setup runs in
        an eager step first."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()  # eager warm-up outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run()
        return self.graph

    def replay(self):
        self.graph.replay()
        return self.out


def capture_steps(steps):
    """Record several steps (e.g. the attention of consecutive layers, each
    with its own cache and weights) into one HIP graph that runs them in
    order, as a whole forward pass would be captured.  Like DecodeStep.capture,
    the graph works on the steps' buffers in place, and one eager pass runs
    first (outside the capture) to do the library's one-time setup."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for st in steps:
            st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for st in steps:
            st.run()
    return graph


class PrefillStep:
    """Device copies of an MLA-form prefill's inputs (padded prompts) and its
    buffers; kv() then attention() (run() does both)."""

    def __init__(self, pf: dict, device: str = "cuda"):
        import torch

        self.torch = torch
        w = pf["workload"]
        self.workload = w
        self.P = int(pf["prompt_len"])
        self.shape = MlaShape.make(
            batch=w.batch, num_heads=w.heads, q_len=1, d_latent=w.d_latent, d_nope=w.d_nope, d_rope=w.d_rope,
            d_v=w.d_v, block_size=w.block_size, max_blocks_per_seq=1, softmax_scale=float(pf["softmax_scale"]))
        bf16 = torch.bfloat16
        self.q_nope = _dev_bits(torch, pf["q_nope"], device, bf16)
        self.q_rope = _dev_bits(torch, pf["q_rope"], device, bf16)
        self.ckr = _dev_bits(torch, pf["ckr"], device, bf16)
        self.w_uk = _dev_bits(torch, pf["w_uk"], device, bf16)
        self.w_uv = _dev_bits(torch, pf["w_uv"], device, bf16)
        self.seq_lens = torch.from_numpy(pf["seq_lens"]).to(device)
        B, P, H = w.batch, self.P, w.heads
        # tile-native per-head keys and values (see mla_prefill_kv)
        n_kv = mla_prefill_kv_elems(self.shape, P)
        self.k_nope = torch.empty(n_kv, dtype=bf16, device=device)
        self.v = torch.empty(n_kv, dtype=bf16, device=device)
        self.out = torch.empty((B, P, H, w.d_v), dtype=bf16, device=device)
        self.lse = torch.empty((B, P, H), dtype=torch.float32, device=device)
        nbytes = mla_prefill_workspace_bytes(self.shape)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)

    def kv(self, stream=None):
        mla_prefill_kv(self.shape, self.P, self.ckr, self.w_uk, self.w_uv, self.seq_lens, self.k_nope, self.v,
                       self.ws, self.ws.numel(), stream)

    def attention(self, stream=None):
        mla_prefill_attention(self.shape, self.P, self.q_nope, self.q_rope, self.k_nope, self.ckr, self.v,
                              self.seq_lens, self.out, self.lse, stream)

    def run(self, stream=None):
        self.kv(stream)
        self.attention(stream)
        return self.out


class TplaStep:
    """The TPLA latent split run on one device: ``n_shards`` decodes over the
    same paged cache, shard i with latent channels [i d_c/n, (i+1) d_c/n), its
    slices of W_UK and W_UV and the whole RoPE key, then the sum of their fp32
    outputs (what the all-reduce would produce).  With ``hadamard`` the cache
    copy held here and the weight slices are first put in the Hadamard basis
    (prepare())."""

    def __init__(self, inputs: dict, n_shards: int = 2, hadamard: bool = True, device: str = "cuda",
                 partial: str = "fp16"):
        import torch

        self.torch = torch
        w = inputs["workload"]
        if w.d_latent % n_shards:
            raise ValueError("d_latent must split evenly over the shards")
        if hadamard and w.cache_dtype != "bf16":
            raise ValueError("the Hadamard basis change needs a bf16 cache")
        self.base = DecodeStep(inputs, device=device, partial=partial)
        self.workload = w
        self.n, self.hadamard = n_shards, bool(hadamard)
        self.num_pages = int(inputs["cache"].shape[0])
        dcs = w.d_latent // n_shards
        self.dcs = dcs
        b = self.base
        self.shard_shape = MlaShape.make(
            batch=w.batch, num_heads=w.heads, q_len=w.q_len, d_latent=dcs, d_nope=w.d_nope, d_rope=w.d_rope,
            d_v=w.d_v, block_size=w.block_size, max_blocks_per_seq=w.max_blocks_per_seq,
            softmax_scale=float(inputs["softmax_scale"]), cache_dtype=b.shape.cache_dtype, out_dtype=MLA_FP32,
            partial_dtype=b.shape.partial_dtype)
        if not combine_up_supported(dcs, w.d_v):
            raise ValueError(f"no merge + up-projection kernel for a {dcs}-wide shard")
        B, S, H = w.batch, w.q_len, w.heads
        bf16, f32 = torch.bfloat16, torch.float32
        self.w_uk_s = torch.empty((n_shards, H, w.d_nope, dcs), dtype=bf16, device=device)
        self.w_uv_s = torch.empty((n_shards, H, dcs, w.d_v), dtype=bf16, device=device)
        self.num_parts = mla_decode_num_parts(self.shard_shape)
        self.q_lat = torch.empty((n_shards, B, S, H, dcs), dtype=bf16, device=device)
        self.o_part = torch.empty((self.num_parts, S * H, dcs), dtype=b.o_part.dtype, device=device)
        self.lse_part = torch.empty((self.num_parts, S * H), dtype=f32, device=device)
        self.parts = torch.empty((n_shards, B, S, H, w.d_v), dtype=f32, device=device)
        self.shard_lse = torch.empty((n_shards, B, S, H), dtype=f32, device=device)
        self.out = b.out  # [B, S_q, H, d_v] in the workload's output type

    def prepare(self, stream=None):
        """Weight slices (in the Hadamard basis if asked) and, then, the cache in that basis."""
        b = self.base
        mla_tpla_split_weights(b.shape, self.n, self.hadamard, b.w_uk, b.w_uv, self.w_uk_s, self.w_uv_s, stream)
        if self.hadamard:
            mla_tpla_rotate_cache(b.shape, b.cache, b.token_stride, b.block_stride, self.num_pages, stream)

    def absorb(self, i: int, stream=None):
        mla_absorb_q(self.shard_shape, self.base.q_nope, self.w_uk_s[i], self.q_lat[i], stream)

    def decode(self, i: int, stream=None):
        """Split-K attention of shard i over its latent channels and the whole RoPE key."""
        b = self.base
        base = b.cache.data_ptr()
        mla_decode_paged(self.shard_shape, self.q_lat[i], b.q_rope, base + i * self.dcs * b.elem,
                         base + self.workload.d_latent * b.elem, b.token_stride, b.block_stride, b.kv_scale,
                         b.block_table, b.seq_lens, self.num_parts, self.o_part, self.lse_part, stream)

    def combine_up(self, i: int, stream=None):
        b = self.base
        mla_combine_up_v(self.shard_shape, self.num_parts, self.o_part, self.lse_part, b.seq_lens, self.w_uv_s[i],
                         self.parts[i], self.shard_lse[i], stream)

    def shard(self, i: int, stream=None):
        """Shard i's decode: its absorbed queries, the split-K attention, the
        merge and its W_UV slice (fp32 into parts[i])."""
        self.absorb(i, stream)
        self.decode(i, stream)
        self.combine_up(i, stream)

    def reduce(self, stream=None):
        mla_tpla_reduce(self.base.shape, self.n, self.parts, self.out, stream)

    def run(self, stream=None):
        for i in range(self.n):
            self.shard(i, stream)
        self.reduce(stream)
        return self.out


class GqaStep:
    """GQLA's GQA decoding path: the latent decode run over per-group records
    [K_nope | V | k_rope], each (sequence, group) stream a sequence of the
    view and the group's heads its rows; the queries [q_nope | 0] are
    regrouped before (mla_gqa_queries) and the value columns of the merged
    rows regrouped after (mla_gqa_output)."""

    def __init__(self, gi: dict, device: str = "cuda", partial: str = "fp16"):
        import torch

        self.torch = torch
        w = gi["workload"]
        G = int(gi["groups"])
        self.workload, self.groups = w, G
        hpg = w.heads // G
        dq = w.d_nope + w.d_v
        common = dict(q_len=w.q_len, d_nope=w.d_nope, d_rope=w.d_rope, d_v=w.d_v, block_size=w.block_size,
                      max_blocks_per_seq=w.max_blocks_per_seq, softmax_scale=float(gi["softmax_scale"]),
                      cache_dtype=MLA_BF16, partial_dtype=MLA_FP16 if partial == "fp16" else MLA_FP32)
        self.shape = MlaShape.make(batch=w.batch, num_heads=w.heads, d_latent=w.d_latent,
                                   out_dtype=MLA_FP32 if w.out_dtype == "fp32" else MLA_BF16, **common)
        self.view = MlaShape.make(batch=w.batch * G, num_heads=hpg, d_latent=dq, out_dtype=MLA_FP32, **common)
        bf16, f32 = torch.bfloat16, torch.float32
        self.q_nope = _dev_bits(torch, gi["q_nope"], device, bf16)
        self.q_rope = _dev_bits(torch, gi["q_rope"], device, bf16)
        self.cache = _dev_bits(torch, gi["cache"], device, bf16)
        self.block_table = torch.from_numpy(gi["block_table"]).to(device)
        self.stream_lens = torch.from_numpy(gi["stream_lens"]).to(device)
        self.token_stride = (dq + w.d_rope) * 2
        self.block_stride = w.block_size * self.token_stride
        self.elem_off = dq * 2
        B, S, H = w.batch, w.q_len, w.heads
        self.q_cat = torch.empty((B * G, S, hpg, dq), dtype=bf16, device=device)
        self.q_rope_g = torch.empty((B * G, S, hpg, w.d_rope), dtype=bf16, device=device)
        self.num_parts = mla_decode_num_parts(self.view)
        self.o_part = torch.empty((self.num_parts, S * hpg, dq), dtype=torch.float16 if partial == "fp16" else f32,
                                  device=device)
        self.lse_part = torch.empty((self.num_parts, S * hpg), dtype=f32, device=device)
        self.o_lat = torch.empty((B * G, S, hpg, dq), dtype=f32, device=device)
        self.lse_g = torch.empty((B * G, S, hpg), dtype=f32, device=device)
        self.out = torch.empty((B, S, H, w.d_v), dtype=f32 if w.out_dtype == "fp32" else bf16, device=device)
        self.lse = torch.empty((B, S, H), dtype=f32, device=device)

    def queries(self, stream=None):
        mla_gqa_queries(self.shape, self.groups, self.q_nope, self.q_rope, self.q_cat, self.q_rope_g, stream)

    def decode(self, stream=None):
        base = self.cache.data_ptr()
        mla_decode_paged(self.view, self.q_cat, self.q_rope_g, base, base + self.elem_off, self.token_stride,
                         self.block_stride, None, self.block_table, self.stream_lens, self.num_parts, self.o_part,
                         self.lse_part, stream)

    def combine(self, stream=None):
        mla_combine_lse(self.view, self.num_parts, self.o_part, self.lse_part, self.stream_lens, self.o_lat,
                        self.lse_g, stream)

    def output(self, stream=None):
        mla_gqa_output(self.shape, self.groups, self.o_lat, self.lse_g, self.out, self.lse, stream)

    def run(self, stream=None):
        self.queries(stream)
        self.decode(stream)
        self.combine(stream)
        self.output(stream)
        return self.out
