"""Float64 NumPy oracle of the per-projection low-rank SwiGLU MLP (test
infrastructure only).

Reading (the alternative wiring of SwiGLU): the MLP sublayer of the LLaMA-2
models the pages pre-train (technical summary §4) keeps its SwiGLU at the full
MLP width f, and each of its three linear maps becomes a low-rank layer of rank
r: a factor into the rank-r space followed by a factor out of it (§1, §2.1),
with nothing between the two factors.  The two input-side layers read the same
normalised input, so their down factors are grouped by concatenation (§2.2,
linear-layer grouping); their up factors have distinct inputs and run as a
batch:

    rstd_t = (sum_j x_tj^2 / d + eps)^(-1/2),   xn = diag(rstd) . x . diag(gamma)
    h_in   = xn . A_in,    A_in = [A_g | A_u]          [T, 2r]
    gate   = h_in[:, :r] . B_g,  up = h_in[:, r:] . B_u  [T, f]
    s      = SiLU(gate) * up                            [T, f]
    h_out  = s . A_o                                    [T, r]
    out    = h_out . B_o   (+ residual)                 [T, d]

Checkpoint (§2.2, low-rank activation checkpointing): the two narrow tensors
h_in and h_out.  The backward recomputes gate, up and s from h_in; in float64
the recomputed values equal the forward ones, so the backward below simply
reuses the forward's.

Everything is float64 with no intermediate rounding; library matmuls are used
as steps and nothing is blocked, fused or reordered.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .block import _dsilu, _f64, _silu, rmsnorm


def mlp_fwd(x, gamma, A_in, B_g, B_u, A_o, B_o, r: int, eps: float, residual=None) -> Dict:
    """Forward of the MLP.  Returns out [T, d], the checkpoint (h_in, h_out),
    the recomputable wide tensors (gate, up, s) and rstd, xn."""
    x, gamma, A_in = _f64(x), _f64(gamma), _f64(A_in)
    xn, _, rstd = rmsnorm(x, gamma, eps)
    h_in = xn @ A_in                                       # grouped down factors
    gate = h_in[:, :r] @ _f64(B_g)                         # batched up factors
    up = h_in[:, r:] @ _f64(B_u)
    s = _silu(gate) * up                                   # SwiGLU at width f
    h_out = s @ _f64(A_o)                                  # output layer: down factor
    out = h_out @ _f64(B_o)                                # and up factor
    if residual is not None:
        out = out + _f64(residual)
    return {"out": out, "h_in": h_in, "h_out": h_out, "gate": gate, "up": up, "s": s,
            "xn": xn, "rstd": rstd}


def mlp_bwd(x, gamma, A_in, B_g, B_u, A_o, B_o, dout, r: int, eps: float, dx_residual=None) -> Dict:
    """Backward for the upstream gradient dout [T, d] (chain rule through the
    forward above).  Returns dx, dgamma, dA_in, dB_g, dB_u, dA_o, dB_o and the
    intermediates dh_out, ds, dgate, dup, dh_in.  `dx_residual`, when given, is
    added to dx (the gradient reaching x through the residual path)."""
    x, gamma, A_in = _f64(x), _f64(gamma), _f64(A_in)
    B_g, B_u, A_o, B_o, dout = _f64(B_g), _f64(B_u), _f64(A_o), _f64(B_o), _f64(dout)
    T, d = x.shape
    f = mlp_fwd(x, gamma, A_in, B_g, B_u, A_o, B_o, r, eps)
    h_in, h_out, gate, up, s = f["h_in"], f["h_out"], f["gate"], f["up"], f["s"]
    xn, rstd = f["xn"], f["rstd"]
    # output layer
    dB_o = h_out.T @ dout
    dh_out = dout @ B_o.T
    dA_o = s.T @ dh_out
    ds = dh_out @ A_o.T
    # SwiGLU at width f
    dgate = ds * up * _dsilu(gate)
    dup = ds * _silu(gate)
    # input layers: batched up factors, then the grouped down factor
    dB_g = h_in[:, :r].T @ dgate
    dB_u = h_in[:, r:].T @ dup
    dh_in = np.concatenate([dgate @ B_g.T, dup @ B_u.T], axis=1)
    dA_in = xn.T @ dh_in
    # RMSNorm
    dxn = dh_in @ A_in.T
    dgamma = np.sum(dxn * x * rstd[:, None], axis=0)
    dot = np.sum(dxn * gamma[None, :] * x, axis=1)         # sum_k gamma_k dxn_tk x_tk
    dx = rstd[:, None] * (gamma[None, :] * dxn - x * (rstd * rstd * dot / d)[:, None])
    if dx_residual is not None:
        dx = dx + _f64(dx_residual)
    return {"dx": dx, "dgamma": dgamma, "dA_in": dA_in, "dB_g": dB_g, "dB_u": dB_u, "dA_o": dA_o,
            "dB_o": dB_o, "dh_out": dh_out, "ds": ds, "dgate": dgate, "dup": dup, "dh_in": dh_in,
            "h_in": h_in, "h_out": h_out, "rstd": rstd}
