"""Helpers for the GPU parity tests: device transfer of generator arrays and the parity
criteria.

Tolerances (fixed by the method's accuracy targets, applied element by element):
  fp32 inputs:  |x - r| <= max(1e-5, 1e-4 |r|)
  bf16 inputs (fp32 accumulation, bf16 outputs):  |x - r| <= 2e-2 max(|r|, rms(r))
  lse (fp32 in every mode): |x - r| <= max(1e-5, 1e-4 |r|); -inf exactly where r = -inf
The rms floor keeps elements whose reference is near zero meaningful in bf16.
"""
import numpy as np
import torch


def dev(x, device="cuda"):
    """numpy generator array -> torch tensor on the GPU (uint16 = bf16 bits)."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, got, ref, dtype, frac_report=None):
    """Assert the parity criterion; returns (max_abs, norm_rel) for reporting."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    if dtype == "f32":
        bound = np.maximum(1e-5, 1e-4 * np.abs(ref))
    else:
        rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
        bound = 2e-2 * np.maximum(np.abs(ref), rms)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} elements out of tolerance; "
                             f"worst at {idx}: got {got[idx]!r} ref {ref[idx]!r}")
    nrm = np.linalg.norm(ref)
    return float(err.max(initial=0.0)), float(np.linalg.norm(got - ref) / nrm) if nrm else 0.0


def check_lse(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), f"{name}: -inf pattern differs"
    g, r = got[~ninf], ref[~ninf]
    assert np.all(np.isfinite(g)), f"{name}: non-finite lse"
    bad = np.abs(g - r) > np.maximum(1e-5, 1e-4 * np.abs(r))
    assert not bad.any(), f"{name}: {bad.sum()} lse values out of tolerance " \
                          f"(max err {np.abs(g - r).max():.3g})"
