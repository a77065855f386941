"""The calibration probes through the C ABI: they run, leave their sinks
untouched (the loads feed a store that never happens) and report rates in
the range a working MI355X gives (sanity bounds, not performance targets)."""
import numpy as np
import pytest

from workloads import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def _time(torch, fn, reps=3):
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    return float(np.median(ts))


def test_hbm_read_probe():
    import torch
    from head_latent_attention_absorbed_amd import mla_probe_hbm_read

    nbytes = 256 << 20
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    t = _time(torch, lambda: mla_probe_hbm_read(x, nbytes, sink))
    gbs = nbytes / t / 1e9
    print(f"[result] hbm read probe {gbs:.0f} GB/s over 256 MiB", flush=True)
    assert 500 < gbs < 9000
    assert int(sink.abs().sum()) == 0


def test_mfma_probe():
    import torch
    from head_latent_attention_absorbed_amd import mla_probe_mfma

    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    flops = {}

    def run():
        flops["n"] = mla_probe_mfma(4000, sink)

    t = _time(torch, run)
    tf = flops["n"] / t / 1e12
    print(f"[result] mfma probe {tf:.0f} TFLOP/s", flush=True)
    assert 200 < tf < 2600
    assert np.isfinite(float(sink[0]))


def test_tile_copy_probe():
    import torch
    from head_latent_attention_absorbed_amd import DecodeStep, mla_probe_tile_copy

    w = small_workload("deepseek_v3", batch=4, seq_len=(700, 2000), max_seq_len=2048, forced_lens=(2000, 1, 0))
    st = DecodeStep(make_inputs(w))
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    base = st.cache.data_ptr()
    mla_probe_tile_copy(st.shape, base, base + w.d_latent * st.elem, st.token_stride, st.block_stride,
                        st.block_table, st.seq_lens, st.num_parts, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
