"""mla_append_kv_noalloc (the library's fixed scratch array, no workspace
argument) against mla_append_kv (caller workspace), through the C ABI.

Two calls in a row share the GPU's one scratch array, the second with a
smaller input, for a bf16 and an e4m3 cache; after each, the whole cache (and
the per-token scales) must equal, bit for bit, what the workspace entry point
writes from the same inputs, and the appended records must match the
oracle's within one step of the stored format.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from workloads import make_append_inputs, make_inputs, small_workload

pytestmark = pytest.mark.gpu

# (first, second): the second call has fewer rows (B * S_q) and a narrower
# hidden state, so it reads a smaller part of the scratch the first call filled.
PAIRS = {
    "bf16": (replace(small_workload("kimi_k2_fp8", batch=12, heads=16, seq_len=(4, 300), max_seq_len=320,
                                    forced_lens=(4, 0, 64, 65, 131)), cache_dtype="bf16", d_model=7168),
             small_workload("deepseek_v3", batch=3, seq_len=(2, 200), max_seq_len=256, forced_lens=(1, 0, 129))),
    "fp8": (small_workload("kimi_k2_fp8", batch=10, heads=16, seq_len=(4, 300), max_seq_len=320,
                           forced_lens=(4, 66, 0, 128)),
            replace(small_workload("deepseek_v3", batch=2, seq_len=(2, 200), max_seq_len=256, forced_lens=(64, 7)),
                    cache_dtype="fp8_e4m3")),
}


def _host(t):
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _append_both(w):
    import torch
    from head_latent_attention_absorbed_amd import DecodeStep

    inputs = make_inputs(w)
    ap = make_append_inputs(w)
    print(f"[case] append_noalloc B={w.batch} S_q={w.q_len} D={w.d_model} cache={w.cache_dtype} "
          f"lens={list(map(int, inputs['seq_lens']))[:8]}", flush=True)
    ref = DecodeStep(inputs)
    ref.set_append_inputs(ap)
    ref.append()
    new = DecodeStep(inputs)
    new.set_append_inputs(ap)
    new.append_ws = None  # the no-allocation call must not need it
    new.append(noalloc=True)
    torch.cuda.synchronize()
    return inputs, ap, ref, new


def _check(w):
    inputs, ap, ref, new = _append_both(w)
    got, want = _host(new.cache), _host(ref.cache)
    assert np.array_equal(got, want), "no-allocation append differs from the workspace append"
    if w.cache_dtype == "fp8_e4m3":
        assert np.array_equal(_host(new.kv_scale), _host(ref.kv_scale), equal_nan=True), "scales differ"
    # and the records are the method's, not just equal to each other
    _, _, positions, rec = oracle.apply_append(inputs, ap)
    bs = w.block_size
    for i, (b, _, p) in enumerate(positions):
        row = got[int(inputs["block_table"][b, p // bs]), p % bs]
        if w.cache_dtype == "bf16":
            vals = oracle.bf16_to_f64(row)
            assert np.all(np.abs(vals - rec[i]) <= 2.0 ** -8 * np.abs(rec[i]) + 1e-6), (b, p)
        else:
            scale = float(_host(new.kv_scale)[int(inputs["block_table"][b, p // bs]), p % bs])
            vals = oracle.e4m3_to_f64(row) * scale
            assert np.all(np.abs(vals - rec[i]) <= 2.0 ** -3 * np.abs(rec[i]) + 2.0 ** -9 * scale), (b, p)


@pytest.mark.parametrize("name", list(PAIRS))
def test_append_noalloc_matches_workspace_append(name):
    first, second = PAIRS[name]
    assert first.batch * first.q_len * first.d_model > second.batch * second.q_len * second.d_model
    _check(first)
    _check(second)
