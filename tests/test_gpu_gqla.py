"""Parity of GQLA's GQA decoding path (mla_gqa_queries, mla_decode_paged and
mla_combine_lse on the per-group view, mla_gqa_output, all through the C
ABI) with the fp64 oracle, at s_q = 2 over paged per-group caches: ragged
and idle sequences, one group (MQA), eight groups (GQA) and one head per
group (MHA), and the LLaMA-3-8B-shaped workload sampled at full size."""
import numpy as np
import pytest

import oracle
from workloads import get_workload, make_gqa_inputs, small_workload
from gpu_helpers import compare, to_np, tolerances

pytestmark = pytest.mark.gpu

SMALL = small_workload("gqla_gqa", batch=4, seq_len=(2, 300), max_seq_len=320, forced_lens=(300, 2, 0, 129),
                       spare_blocks=3)


def _run(gi):
    import torch
    from head_latent_attention_absorbed_amd import GqaStep

    st = GqaStep(gi)
    st.out.fill_(float("nan"))
    st.run()
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("groups", [8, 1, 32])
def test_gqa_path_parity(groups):
    gi = make_gqa_inputs(SMALL, groups)
    print(f"[case] gqa path groups={groups} lens={list(gi['seq_lens'])}", flush=True)
    st = _run(gi)
    ref = oracle.gqa_decode(gi)
    tol_abs, tol_rel = tolerances(SMALL)
    compare("out", to_np(st.out), ref["out"], tol_abs, tol_rel)
    compare("lse", to_np(st.lse), ref["lse"], tol_abs, tol_rel, finite_only=True)


def test_gqa_path_full_workload_sampled():
    """B = 16, H = 32 in 8 groups, s_q = 2, context 8192: sampled sequences
    and heads (both queries) against the oracle, every output finite."""
    w = get_workload("gqla_gqa")
    gi = make_gqa_inputs(w, 8)
    print("[case] gqa path full workload", flush=True)
    st = _run(gi)
    out = to_np(st.out)
    assert np.all(np.isfinite(out))
    batches, heads = [0, 9, 15], [0, 3, 4, 17, 31]
    ref = oracle.gqa_decode(gi, batches=batches, heads=heads)
    tol_abs, tol_rel = tolerances(w)
    compare("out sampled", out[batches][:, :, heads], ref["out"], tol_abs, tol_rel)


def test_gqa_path_fp32_out():
    from dataclasses import replace

    w = replace(SMALL, out_dtype="fp32")
    gi = make_gqa_inputs(w, 8)
    print("[case] gqa path fp32 out", flush=True)
    st = _run(gi)
    assert str(st.out.dtype) == "torch.float32"
    ref = oracle.gqa_decode(gi)
    tol_abs, tol_rel = tolerances(w)
    compare("out", to_np(st.out), ref["out"], tol_abs, tol_rel)
