"""Shared helpers of the GPU tests: run one step through the C ABI, compare."""
import math

import numpy as np

TOL_ABS = 1e-2
TOL_REL = 5e-3


def tolerances(workload):
    """max |err| <= 1e-2 and relative L2 <= 5e-3 for bf16 inputs with fp32
    accumulation, twice that when the cache is e4m3."""
    k = 2.0 if workload.cache_dtype == "fp8_e4m3" else 1.0
    return TOL_ABS * k, TOL_REL * k


def to_np(t):
    import torch

    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def compare(name, got, ref, tol_abs, tol_rel, finite_only=False, scaled_abs=True):
    """max |err| and relative L2 over the tensor.  With scaled_abs the
    element bound is tol_abs * max(1, |ref|): a bf16 result carries a rounding
    error of up to 2^-9 |ref|, more than 1e-2 once |ref| > 2.56 (edge cases
    such as one-token sequences return raw value rows); for |ref| <= 1, the
    range of every named workload's outputs, it is the plain bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    if finite_only:
        # -inf entries must agree exactly; the rest are compared numerically
        inf_ref = np.isneginf(ref)
        assert np.array_equal(np.isneginf(got), inf_ref), f"{name}: -inf pattern differs"
        got, ref = got[~inf_ref], ref[~inf_ref]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if got.size == 0:
        return 0.0, 0.0
    err = np.abs(got - ref)
    max_abs = float(err.max())
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / denom) if denom > 0 else float(np.linalg.norm(got - ref))
    bound = tol_abs * np.maximum(1.0, np.abs(ref)) if scaled_abs else tol_abs
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"{name}: max abs err {max_abs:.3e} exceeds {tol_abs:.1e}{' x max(1,|ref|)' if scaled_abs else ''} (rel L2 {rel:.3e})"
    assert rel <= tol_rel, f"{name}: rel L2 {rel:.3e} > {tol_rel:.1e} (max abs {max_abs:.3e})"
    return max_abs, rel


GUARD_ELEMS = 256  # guard elements before and after each output (>= 16 bytes, keeps alignment)


def _guarded(t):
    """A copy of tensor t's shape and dtype inside a larger allocation with
    GUARD_ELEMS elements before and after it, filled with a sentinel pattern.
    Returns (view, guards)."""
    import torch

    base = torch.empty(t.numel() + 2 * GUARD_ELEMS, dtype=t.dtype, device=t.device)
    base.view(torch.uint8).fill_(0xA5)
    view = base[GUARD_ELEMS: GUARD_ELEMS + t.numel()].view(t.shape)
    return view, (base[:GUARD_ELEMS], base[GUARD_ELEMS + t.numel():])


def run_step(inputs, num_parts=None, poison=True, partial="fp16", fused=None, guard=True):
    """One step through the C ABI; ``fused`` None takes the step's default
    (merge and up-projection in one launch where a kernel exists).  With
    ``guard`` every buffer the step writes sits between two guard regions of
    a sentinel byte pattern, which must be untouched afterwards (writes stay
    inside their tensors)."""
    import torch
    from head_latent_attention_absorbed_amd import DecodeStep

    st = DecodeStep(inputs, num_parts=num_parts, partial=partial, fused=fused)
    guards = {}
    if guard:
        for name in ("q_lat", "o_part", "lse_part", "o_lat", "lse", "out"):
            t = getattr(st, name)
            if t is not None:
                view, g = _guarded(t)
                setattr(st, name, view)
                guards[name] = g
    if poison:
        for t in (st.q_lat, st.o_part, st.lse_part, st.o_lat, st.lse, st.out):
            if t is not None:
                t.fill_(float("nan"))
    st.run()
    torch.cuda.synchronize()
    for name, (lo, hi) in guards.items():
        for side, g in (("before", lo), ("after", hi)):
            bytes_ = g.view(torch.uint8).cpu().numpy()
            assert np.all(bytes_ == 0xA5), f"{name}: {np.count_nonzero(bytes_ != 0xA5)} guard bytes {side} it changed"
    return st
