"""mla_validate_decode_inputs on the GPU: the generated inputs (idle slots,
ragged lengths, a random page permutation, -1 entries past each sequence's
pages) count no violation, and each planted violation counts exactly once."""
import numpy as np
import pytest

from workloads import make_inputs, small_workload

pytestmark = pytest.mark.gpu

W = small_workload("deepseek_v3", batch=4, heads=16, seq_len=(1, 300), max_seq_len=320,
                   forced_lens=(0, 1, 130, 300), spare_blocks=2)


def _count(inputs, lens=None, table=None, num_pages=None, q_len=None):
    import torch
    from head_latent_attention_absorbed_amd import DecodeStep, mla_validate_decode_inputs

    st = DecodeStep(inputs)
    if q_len is not None:
        st.shape.q_len = q_len
    bt = st.block_table if table is None else torch.from_numpy(table).to("cuda")
    sl = st.seq_lens if lens is None else torch.from_numpy(lens).to("cuda")
    pages = inputs["cache"].shape[0] if num_pages is None else num_pages
    out = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    mla_validate_decode_inputs(st.shape, bt, sl, pages, out)
    torch.cuda.synchronize()
    return int(out.item())


def test_generated_inputs_are_valid():
    inputs = make_inputs(W)
    print(f"[case] validate generated lens={list(inputs['seq_lens'])}", flush=True)
    assert _count(inputs) == 0


def test_planted_violations_count_once_each():
    inputs = make_inputs(W)
    print("[case] validate planted", flush=True)
    lens = inputs["seq_lens"].copy()
    table = inputs["block_table"].copy()
    pages = inputs["cache"].shape[0]
    bs = W.block_size
    # a page id past the cache inside sequence 3's pages, and a -1 inside sequence 2's
    table[3, (int(lens[3]) - 1) // bs] = pages
    table[2, 0] = -1
    assert _count(inputs, table=table) == 2
    # entries past a sequence's pages are not read
    table = inputs["block_table"].copy()
    table[1, 1:] = -5
    assert _count(inputs, table=table) == 0
    # a length longer than the table can hold; a negative length
    bad = lens.copy()
    bad[2] = W.max_blocks_per_seq * bs + 1
    bad[0] = -3
    assert _count(inputs, lens=bad) == 2
    # with 2 queries per sequence, the one-token sequence is too short
    assert _count(inputs, q_len=2) == 1
    # fewer pages than the table refers to
    used = max(int(table[b, i]) for b in range(W.batch) for i in range((int(lens[b]) + bs - 1) // bs))
    assert _count(inputs, num_pages=used) >= 1
