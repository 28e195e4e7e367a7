"""Float64 NumPy oracle of the low-rank bottleneck block (test infrastructure only).

Notation follows the BOOST pages: T = b*s tokens, hidden width d, rank r.  A
low-rank layer replaces a d x d weight by a d x r "down" factor followed by an
r x d "up" factor with operations between them (technical summary §1 and §2.1).
Down-projections that read the same input are grouped by concatenating their
weights; up-projections with distinct inputs run as a batch (§2.2, "linear
layer grouping").  So with g grouped branches:

    A   = [A_0 | A_1 | ... | A_{g-1}]            [d, g*r]   (branch-major columns)
    B_i                                         [r, d]     for i < n_up

Block (reading: pre-norm, sigma between the two projections, no bias, no
residual):

    rstd_t = (sum_j x_tj^2 / D + eps)^(-1/2)     D = d, or the unsharded width
    xn     = diag(rstd) . x . diag(gamma)
    h      = xn . A                               [T, g*r]  (the rank-r checkpoint)
    z_i    = sigma(h_i)                           identity | SiLU
             SiLU(h_0) * h_1                      SwiGLU (g = 2, n_up = 1)
    y_i    = z_i . B_i                            [T, d]

Everything is float64 with no intermediate rounding; library matmuls are used as
steps and nothing is blocked, fused or reordered.  ``working_precision`` runs the
same code in another NumPy float type (float32 for the CPU speed baseline); the
tests and the parity checks use the float64 default.

Residual variant (reading: the block is the body of a pre-norm transformer
sublayer of the LLaMA-2 models the pages train, technical summary §4, whose
output adds the sublayer's input back):

    y_i    = residual_i + z_i . B_i              (residual_i [T, d], given)
    dx     = (the block's dx) + dx_residual      (dx_residual [T, d], given: the
                                                   gradient reaching x through the
                                                   residual path, e.g. dy_0 when
                                                   residual_0 = x)
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import contextlib

import numpy as np

_DTYPE = np.float64


@contextlib.contextmanager
def working_precision(dtype):
    """Run the oracle's arithmetic in `dtype` (np.float64 by default) inside the
    block; the formulas are unchanged, only the arrays' float type."""
    global _DTYPE
    old, _DTYPE = _DTYPE, np.dtype(dtype).type
    try:
        yield
    finally:
        _DTYPE = old


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=_DTYPE)


def branch_slices(r: int, g: int) -> List[slice]:
    """Column range of branch i inside the concatenated [d, g*r] weight and the
    [T, g*r] pre-activation (branch-major concatenation, §2.2 grouping)."""
    return [slice(i * r, (i + 1) * r) for i in range(g)]


# ----------------------------------------------------------------------------- sigma
def _sigmoid(v: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-v))


def _silu(v: np.ndarray) -> np.ndarray:
    return v * _sigmoid(v)


def _dsilu(v: np.ndarray) -> np.ndarray:
    s = _sigmoid(v)
    return s * (1.0 + v * (1.0 - s))


def act_forward(h: np.ndarray, act: str, r: int, g: int) -> List[np.ndarray]:
    """The pointwise operation at rank r between the projections (§2.1 calls
    them the intermediate operations on the narrow activation).  Reading:
    identity for a plain factorisation, SiLU for a CoLA-style bottleneck, and
    SwiGLU = SiLU(gate) * up for a grouped gate/up pair."""
    h = _f64(h)
    hs = [h[:, s] for s in branch_slices(r, g)]
    if act == "identity":
        return [hi.copy() for hi in hs]
    if act == "silu":
        return [_silu(hi) for hi in hs]
    if act == "swiglu":
        if g != 2:
            raise ValueError("swiglu needs g == 2 (gate, up)")
        return [_silu(hs[0]) * hs[1]]
    raise ValueError(act)


def act_backward(h: np.ndarray, dz: Sequence[np.ndarray], act: str, r: int, g: int) -> np.ndarray:
    """Chain rule through sigma: returns dh [T, g*r] from dz_i [T, r]."""
    h = _f64(h)
    hs = [h[:, s] for s in branch_slices(r, g)]
    dh = np.empty_like(h)
    sl = branch_slices(r, g)
    if act == "identity":
        for i in range(g):
            dh[:, sl[i]] = dz[i]
    elif act == "silu":
        for i in range(g):
            dh[:, sl[i]] = dz[i] * _dsilu(hs[i])
    elif act == "swiglu":
        dh[:, sl[0]] = dz[0] * hs[1] * _dsilu(hs[0])
        dh[:, sl[1]] = dz[0] * _silu(hs[0])
    else:
        raise ValueError(act)
    return dh


# ----------------------------------------------------------------------------- RMSNorm
def rms_stats(x: np.ndarray, D: int, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token statistic of RMSNorm (§2.2 "Online-RMSNorm": the statistic is a
    sum of squares, computed locally and applied later).  Reading: eps inside
    the square root, mean over D.  Returns (sum of squares, rstd)."""
    x = _f64(x)
    ss = np.sum(x * x, axis=1)
    rstd = 1.0 / np.sqrt(ss / D + eps)
    return ss, rstd


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, D: int = 0):
    """RMSNorm(x) = x * rstd * gamma, gamma applied after normalisation.
    Returns (y, ss, rstd)."""
    x = _f64(x)
    D = D or x.shape[1]
    ss, rstd = rms_stats(x, D, eps)
    return x * rstd[:, None] * _f64(gamma)[None, :], ss, rstd


# ----------------------------------------------------------------------------- block
def block_fwd(x, gamma, A, B: Sequence, r: int, g: int, act: str, eps: float, D: int = 0,
              residual: Sequence = None) -> Dict:
    """Forward of the block.  Returns y (list of [T, d]), h (the checkpoint),
    z (list), xn and rstd.  With `residual` (a list of n_up [T, d] arrays),
    y_i = residual_i + z_i . B_i."""
    x, gamma, A = _f64(x), _f64(gamma), _f64(A)
    xn, ss, rstd = rmsnorm(x, gamma, eps, D)
    h = xn @ A                                           # grouped down-projection
    z = act_forward(h, act, r, g)
    y = [zi @ _f64(Bi) for zi, Bi in zip(z, B)]          # batched up-projection
    if residual is not None:
        if len(residual) != len(y):
            raise ValueError("one residual per up-projection")
        y = [yi + _f64(ri) for yi, ri in zip(y, residual)]
    return {"y": y, "h": h, "z": z, "xn": xn, "rstd": rstd, "ss": ss}


def block_bwd(x, gamma, A, B: Sequence, dy: Sequence, r: int, g: int, act: str, eps: float,
              D: int = 0, dx_residual=None) -> Dict:
    """Backward of the block for upstream gradients dy_i.  The activation is
    recomputed from the rank-r pre-activation h (§2.2 "low-rank activation
    checkpointing": only the narrow tensor is kept); in float64 the recomputed
    h equals the forward one.  Returns dx, dgamma, dA, dB (list) and the
    intermediates dz, dh, dxn.  `dx_residual` ([T, d]), when given, is added to
    dx: the gradient that reaches x through the residual path (the residual
    added in the forward does not change dB, dz or anything upstream of y)."""
    x, gamma, A = _f64(x), _f64(gamma), _f64(A)
    T, d = x.shape
    D = D or d
    f = block_fwd(x, gamma, A, B, r, g, act, eps, D)
    h, z, xn, rstd = f["h"], f["z"], f["xn"], f["rstd"]
    dy = [_f64(t) for t in dy]
    dB = [zi.T @ dyi for zi, dyi in zip(z, dy)]
    dz = [dyi @ _f64(Bi).T for dyi, Bi in zip(dy, B)]
    dh = act_backward(h, dz, act, r, g)
    dA = xn.T @ dh
    dxn = dh @ A.T
    dgamma = np.sum(dxn * x * rstd[:, None], axis=0)
    dot = np.sum(dxn * gamma[None, :] * x, axis=1)       # sum_k gamma_k dxn_tk x_tk
    dx = rstd[:, None] * (gamma[None, :] * dxn - x * (rstd * rstd * dot / D)[:, None])
    if dx_residual is not None:
        dx = dx + _f64(dx_residual)
    return {"dx": dx, "dgamma": dgamma, "dA": dA, "dB": dB, "dz": dz, "dh": dh, "dxn": dxn,
            "h": h, "rstd": rstd}


# ----------------------------------------------------------------------------- shard seam
def down_partial(x_s, gamma_s, A_s) -> Tuple[np.ndarray, np.ndarray]:
    """One tensor-parallel shard's half of the block under bottleneck-aware TP
    (§2.1: the d x r factor runs row-parallel over a slice of d, so its output
    is a partial sum over the shard; §2.2: Online-RMSNorm keeps only the local
    sum of squares and defers normalisation).  Returns the un-normalised
    partial (x_s * gamma_s) . A_s and the local sum of squares."""
    x_s = _f64(x_s)
    part = (x_s * _f64(gamma_s)[None, :]) @ _f64(A_s)
    ss = np.sum(x_s * x_s, axis=1)
    return part, ss


def up_finish(partial, ss, B_s: Sequence, r: int, g: int, act: str, eps: float, D: int) -> Dict:
    """Second half of the seam, after the (here: absent) all-reduce of the
    partial and the statistic: apply the deferred normalisation with the
    global width D, sigma, then the column-parallel r x d factor on this
    shard's columns.  Returns y (list) and h."""
    partial, ss = _f64(partial), _f64(ss)
    rstd = 1.0 / np.sqrt(ss / D + eps)
    h = partial * rstd[:, None]
    z = act_forward(h, act, r, g)
    y = [zi @ _f64(Bi) for zi, Bi in zip(z, B_s)]
    return {"y": y, "h": h, "z": z, "rstd": rstd}
