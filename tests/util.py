"""Helpers shared by the tests: moving seeded inputs to the GPU, the
tolerance check and the MLP's selection-case inputs.  Holds none of the
method's arithmetic."""
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


def mlp_selection_case(T=5, d=8, f=6, r=3, seed=0):
    """Inputs of the per-projection MLP's selection case (arrays only): x in
    {+-1}, gamma = 1; one-hot A_in columns select coordinates sel_g (gate half)
    and sel_u (up half); B_g = B_u = [I_r | 0]; A_o = [I_r ; 0]; B_o sends rank
    index k to coordinate sel_o[k].  Returns (x, gamma, A_in, B_g, B_u, A_o,
    B_o, sel_g, sel_u, sel_o)."""
    rng = np.random.default_rng(seed)
    x = np.where(rng.random((T, d)) < 0.5, -1.0, 1.0)
    sel_g, sel_u, sel_o = rng.permutation(d)[:r], rng.permutation(d)[:r], rng.permutation(d)[:r]
    A_in = np.zeros((d, 2 * r))
    A_in[sel_g, np.arange(r)] = 1.0
    A_in[sel_u, r + np.arange(r)] = 1.0
    B_g = np.zeros((r, f))
    B_g[np.arange(r), np.arange(r)] = 1.0
    B_u = B_g.copy()
    A_o = np.zeros((f, r))
    A_o[np.arange(r), np.arange(r)] = 1.0
    B_o = np.zeros((r, d))
    B_o[np.arange(r), sel_o] = 1.0
    return x, np.ones(d), A_in, B_g, B_u, A_o, B_o, sel_g, sel_u, sel_o
