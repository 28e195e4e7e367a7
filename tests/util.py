"""Helpers shared by the tests: moving seeded inputs to the GPU and the
tolerance check.  Holds none of the block's arithmetic."""
from __future__ import annotations

import numpy as np
import torch

# bf16: fp32 accumulation, outputs rounded once to bf16; fp32: plain fp32 arithmetic
TOL = {"bf16": (1e-2, 5e-3), "f32": (1e-5, 1e-5)}   # (max |e| / max |ref|, ||e||_F / ||ref||_F)


def dev(t, device="cuda"):
    """A workloads.Tensor (or ndarray of float32) -> torch tensor on the GPU."""
    store = t.store if hasattr(t, "store") else t
    if store.dtype == np.uint16:
        return torch.from_numpy(store.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(store)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    e = got - ref
    mx = np.max(np.abs(e)) / max(np.max(np.abs(ref)), 1e-300)
    fr = np.linalg.norm(e) / max(np.linalg.norm(ref), 1e-300)
    return mx, fr


def assert_close(got, ref, dtype: str, what: str = ""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    mx, fr = errors(got, ref)
    tmax, tfr = TOL[dtype]
    assert mx <= tmax and fr <= tfr, f"{what}: max rel {mx:.3e} (<= {tmax}), frob rel {fr:.3e} (<= {tfr})"
    return mx, fr
