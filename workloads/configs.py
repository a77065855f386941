"""The five decode workloads and the knobs of smaller parity cases.

Shapes follow the absorbed Multi-Head Latent Attention decode the pages
describe: a per-token latent c_KV of rank d_c plus a decoupled RoPE key of
width d_r that every head shares (the MQA form named in the GQLA abstract on
the "GQA-to-MLA" Daily Papers listing), per-head W_UK [d_n, d_c] and
W_UV [d_c, d_v].  The 576-value record of the bf16 workloads equals 7.03 %
of LLaMA-2-7B's 8192 values per token per layer, the KV size the TransMLA
review page (core_discovery) reports after conversion.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    q_len: int
    d_latent: int
    seq_len: Tuple[int, int]          # inclusive range of integer lengths
    paged: bool                       # False: identity block table (contiguous)
    cache_dtype: str                  # "bf16" or "fp8_e4m3"
    out_dtype: str                    # "bf16" or "fp32"
    weight_var: float                 # variance of W_UK / W_UV entries
    seed: int
    d_nope: int = 128
    d_rope: int = 64
    d_v: int = 128
    block_size: int = 64
    # Width of the hidden state the cache append projects from (the
    # MHA-converted 7B model's 4096 = 32 heads x 128).
    d_model: int = 4096
    # Largest length the block table has room for (defaults to seq_len[1]).
    max_seq_len: Optional[int] = None
    # Extra unused physical pages beyond those the sequences need.
    spare_blocks: int = 0
    # Lengths forced for the first few sequences (edge cases), then drawn.
    forced_lens: Tuple[int, ...] = field(default_factory=tuple)
    description: str = ""

    @property
    def softmax_scale(self) -> float:
        # The score is a dot product over the d_nope + d_rope query/key width,
        # which the latent split does not change.
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)

    @property
    def capacity(self) -> int:
        return self.max_seq_len if self.max_seq_len is not None else self.seq_len[1]

    @property
    def max_blocks_per_seq(self) -> int:
        return max(1, -(-self.capacity // self.block_size))

    @property
    def record_elems(self) -> int:
        return self.d_latent + self.d_rope


WORKLOADS = {
    "tiny": Workload(
        name="tiny", batch=1, heads=16, q_len=1, d_latent=512, seq_len=(1024, 1024),
        paged=False, cache_dtype="bf16", out_dtype="bf16", weight_var=1.0 / 512, seed=1000,
        description="Tiny MLA decode: B=1, H=16, 1 query token, context 1024, contiguous cache",
    ),
    "deepseek_v3": Workload(
        name="deepseek_v3", batch=32, heads=128, q_len=1, d_latent=512, seq_len=(4096, 8192),
        paged=True, cache_dtype="bf16", out_dtype="bf16", weight_var=1.0 / 512, seed=1001,
        description="DeepSeek-V3-shaped decode: B=32, H=128, seq_lens uniform in [4096, 8192], paged 64",
    ),
    "gqa7b": Workload(
        name="gqa7b", batch=16, heads=32, q_len=1, d_latent=512, seq_len=(8192, 8192),
        paged=True, cache_dtype="bf16", out_dtype="bf16", weight_var=1.0 / 512, seed=1002,
        description="GQA-converted 7B-shaped MLA: B=16, H=32, context 8192, paged 64",
    ),
    "tpla_shard": Workload(
        name="tpla_shard", batch=8, heads=128, q_len=1, d_latent=256, seq_len=(32768, 32768),
        paged=True, cache_dtype="bf16", out_dtype="fp32", weight_var=1.0 / 256, seed=1003,
        description="One latent-split TP shard: B=8, H=128, d_c=256, context 32768, fp32 partial out + LSE",
    ),
    "gqla_gqa": Workload(
        name="gqla_gqa", batch=16, heads=32, q_len=2, d_latent=512, seq_len=(8192, 8192),
        paged=True, cache_dtype="bf16", out_dtype="bf16", weight_var=1.0 / 512, seed=1005,
        description="GQLA's two decoding paths at s_q = 2 for a LLaMA-3-8B-shaped model: B=16, H=32 in 8 "
                    "groups, context 8192 (MQA-absorb over the latent, or GQA over per-group K/V)",
    ),
    "kimi_k2_fp8": Workload(
        name="kimi_k2_fp8", batch=16, heads=64, q_len=4, d_latent=512, seq_len=(16384, 32768),
        paged=True, cache_dtype="fp8_e4m3", out_dtype="bf16", weight_var=1.0 / 512, seed=1004,
        description="Kimi-K2-shaped 4-token causal decode over an e4m3 cache with per-token fp32 scale",
    ),
}

# The order of the workloads; the seed of workload i is 1000 + i.
WORKLOAD_ORDER = ("tiny", "deepseek_v3", "gqa7b", "tpla_shard", "kimi_k2_fp8", "gqla_gqa")


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def small_workload(base: str, **overrides) -> Workload:
    """A reduced copy of a named workload (same dtypes and head dims)."""
    w = get_workload(base)
    overrides.setdefault("name", f"{base}_small")
    return replace(w, **overrides)


PREFILL_PROMPT_LEN = 4096


def prefill_workload() -> tuple[Workload, int]:
    """The prompt batch of the prefill measurement: DeepSeek-V3 heads
    (H = 128, d_c = 512, d_nope = d_v = 128), two prompts padded to 4096
    positions, the first full and the second of a length drawn from
    [2048, 4096].  Returns (workload, padded prompt length)."""
    w = replace(get_workload("deepseek_v3"), name="deepseek_v3_prefill", batch=2, seq_len=(2048, PREFILL_PROMPT_LEN),
                forced_lens=(PREFILL_PROMPT_LEN,))
    return w, PREFILL_PROMPT_LEN


# Key/value groups of the GQLA workload (LLaMA-3-8B: 32 query heads, 8 KV heads).
GQLA_GROUPS = 8
