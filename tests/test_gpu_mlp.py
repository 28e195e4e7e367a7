"""Parity of the per-projection low-rank SwiGLU MLP (lr_mlp_fwd / lr_mlp_bwd
through the C ABI) with the CPU oracle (oracle/mlp.py).

Small cases compare every output and gradient whole and span several tiles
with ragged tails (T, and MLP widths f that leave a partial last column tile);
the mid-size case has the full widths, so its weight gradients run the same
plans as the full size (one token pass for the output layer's 236 tiles and
the input layers' 472); the full-size case compares sampled rows of out, the
checkpoint and dx (rows are independent in all three).  Tolerances as for the block:
bf16 max|e| <= 1e-2 max|ref| and ||e||_F <= 5e-3 ||ref||_F; fp32 1e-5.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import rank_bottleneck_amd as rb
from workloads import MLP_WORKLOADS, MlpWorkload, make_mlp_inputs

from util import assert_close, dev, host, mlp_selection_case

pytestmark = pytest.mark.gpu

GRADS = ("dx", "dgamma", "dA_in", "dB_g", "dB_u", "dA_o", "dB_o")


def _say(*a):
    print("[gpu-mlp]", *a, file=sys.stderr, flush=True)


def _dims(wl, T=None):
    return rb.make_mlp_dims(wl.T if T is None else T, wl.d, wl.f, wl.r, wl.dtype, wl.eps)


def _weights(inp):
    return [dev(t) for t in (inp.gamma, inp.A_in, inp.B_g, inp.B_u, inp.A_o, inp.B_o)]


def _wv(inp):
    return [t.v for t in (inp.gamma, inp.A_in, inp.B_g, inp.B_u, inp.A_o, inp.B_o)]


def _sample_rows(T, n=1024, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.choice(T, n - 8, replace=False), np.arange(T - 8, T)]))


SMALL = [
    MlpWorkload("mlp_f32_tiny", T=130, d=128, f=192, r=64, dtype="f32"),
    # fp32 over several 128 x 128 tiles in every GEMM, with the residual
    MlpWorkload("mlp_f32_res", T=300, d=256, f=320, r=128, dtype="f32", residual=True),
    MlpWorkload("mlp_bf16_ragged", T=555, d=320, f=448, r=128, dtype="bf16"),
    MlpWorkload("mlp_bf16_res", T=300, d=256, f=704, r=64, dtype="bf16", residual=True),
    MlpWorkload("mlp_bf16_r192", T=777, d=512, f=576, r=192, dtype="bf16"),
    MlpWorkload("mlp_bf16_256tiles", T=1100, d=1024, f=1344, r=256, dtype="bf16", residual=True),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_mlp_forward_backward_small(wl):
    _say("small", wl)
    inp = make_mlp_inputs(wl, seed=1)
    dims = _dims(wl)
    x = dev(inp.x)
    w = _weights(inp)
    rstd = torch.empty(wl.T, dtype=torch.float32, device="cuda")
    out, h_in, h_out = rb.mlp_fwd(dims, x, *w, residual=x if wl.residual else None, rstd=rstd)
    torch.cuda.synchronize()
    ref = oracle.mlp_fwd(inp.x.v, *_wv(inp), wl.r, wl.eps, residual=inp.x.v if wl.residual else None)
    assert_close(host(h_in), ref["h_in"], wl.dtype, "h_in")
    assert_close(host(h_out), ref["h_out"], wl.dtype, "h_out")
    assert_close(host(out), ref["out"], wl.dtype, "out")
    assert_close(host(rstd), ref["rstd"], "f32", "rstd")
    dout = dev(inp.dout)
    # the saved rstd, and rstd recomputed from x
    for rs in (rstd, None):
        g = rb.mlp_bwd(dims, x, *w, h_in, h_out, dout, rstd=rs, dx_residual=dout if wl.residual else None)
        torch.cuda.synchronize()
        rg = oracle.mlp_bwd(inp.x.v, *_wv(inp), inp.dout.v, wl.r, wl.eps,
                            dx_residual=inp.dout.v if wl.residual else None)
        for k in GRADS:
            assert_close(host(g[k]), rg[k], wl.dtype, k)


def test_mlp_in_place_residuals():
    """residual == out in the forward and dx_residual == dx in the backward (the
    residual stream updated in place)."""
    wl = MlpWorkload("mlp_inplace", T=333, d=256, f=448, r=64, dtype="bf16")
    _say("in place", wl)
    inp = make_mlp_inputs(wl, seed=4)
    dims = _dims(wl)
    x = dev(inp.x)
    w = _weights(inp)
    out = x.clone()
    h_in = torch.empty(wl.T, 2 * wl.r, dtype=torch.bfloat16, device="cuda")
    h_out = torch.empty(wl.T, wl.r, dtype=torch.bfloat16, device="cuda")
    ws = rb.mlp_workspace(dims, False)
    rb.lr_mlp_fwd(dims, x, *w, out, out, h_in, h_out, None, ws)
    dout = dev(inp.dout)
    dx = dout.clone()
    f32 = dict(dtype=torch.float32, device="cuda")
    gr = [torch.empty(wl.d, **f32), torch.empty(wl.d, 2 * wl.r, **f32), torch.empty(wl.r, wl.f, **f32),
          torch.empty(wl.r, wl.f, **f32), torch.empty(wl.f, wl.r, **f32), torch.empty(wl.r, wl.d, **f32)]
    rb.lr_mlp_bwd(dims, x, *w, h_in, h_out, None, dout, dx, dx, *gr, rb.mlp_workspace(dims, True))
    torch.cuda.synchronize()
    ref = oracle.mlp_fwd(inp.x.v, *_wv(inp), wl.r, wl.eps, residual=inp.x.v)
    assert_close(host(out), ref["out"], wl.dtype, "out (in place)")
    rg = oracle.mlp_bwd(inp.x.v, *_wv(inp), inp.dout.v, wl.r, wl.eps, dx_residual=inp.dout.v)
    assert_close(host(dx), rg["dx"], wl.dtype, "dx (in place)")
    for k, t in zip(GRADS[1:], gr):
        assert_close(host(t), rg[k], wl.dtype, k)


def test_mlp_no_rows():
    """T = 0: nothing to normalise, every weight gradient is zero."""
    wl = MlpWorkload("mlp_empty", T=0, d=128, f=192, r=64, dtype="bf16")
    inp = make_mlp_inputs(wl.replace(T=4), seed=5)
    dims = _dims(wl)
    w = _weights(inp)
    x = torch.empty(0, wl.d, dtype=torch.bfloat16, device="cuda")
    out, h_in, h_out = rb.mlp_fwd(dims, x, *w)
    g = rb.mlp_bwd(dims, x, *w, h_in, h_out, torch.empty(0, wl.d, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, wl.d)
    for k in GRADS[1:]:
        assert torch.count_nonzero(g[k]).item() == 0, k


def test_mlp_full_widths_whole_gradients():
    """The full widths (d = 4096, f = 11008, r = 1024) at T = 4096: the weight
    gradients run the full size's plans; every output and gradient whole."""
    wl = MLP_WORKLOADS["lowrank_mlp"].replace(T=4096)
    _say("full widths", wl)
    inp = make_mlp_inputs(wl, seed=2)
    dims = _dims(wl)
    x = dev(inp.x)
    w = _weights(inp)
    out, h_in, h_out = rb.mlp_fwd(dims, x, *w, residual=x)
    dout = dev(inp.dout)
    g = rb.mlp_bwd(dims, x, *w, h_in, h_out, dout, dx_residual=dout)
    torch.cuda.synchronize()
    ref = oracle.mlp_fwd(inp.x.v, *_wv(inp), wl.r, wl.eps, residual=inp.x.v)
    assert_close(host(out), ref["out"], wl.dtype, "out")
    assert_close(host(h_in), ref["h_in"], wl.dtype, "h_in")
    assert_close(host(h_out), ref["h_out"], wl.dtype, "h_out")
    rg = oracle.mlp_bwd(inp.x.v, *_wv(inp), inp.dout.v, wl.r, wl.eps, dx_residual=inp.dout.v)
    for k in GRADS:
        assert_close(host(g[k]), rg[k], wl.dtype, k)


def test_mlp_full_size_sampled_rows():
    """The benchmark's shape and calls (T = 16384): out, h_in, h_out and dx on
    1024 sampled rows (the last 8 included), each row's values computed by the
    oracle from that row alone."""
    wl = MLP_WORKLOADS["lowrank_mlp"]
    _say("full size", wl)
    inp = make_mlp_inputs(wl, seed=0)
    dims = _dims(wl)
    x = dev(inp.x)
    w = _weights(inp)
    rstd = torch.empty(wl.T, dtype=torch.float32, device="cuda")
    out, h_in, h_out = rb.mlp_fwd(dims, x, *w, residual=x, rstd=rstd)
    dout = dev(inp.dout)
    g = rb.mlp_bwd(dims, x, *w, h_in, h_out, dout, rstd=rstd, dx_residual=dout)
    torch.cuda.synchronize()
    rows = _sample_rows(wl.T)
    ri = torch.as_tensor(rows, device="cuda")
    xv = inp.x.v[rows]
    ref = oracle.mlp_fwd(xv, *_wv(inp), wl.r, wl.eps, residual=xv)
    assert_close(host(out[ri]), ref["out"], wl.dtype, "out rows")
    assert_close(host(h_in[ri]), ref["h_in"], wl.dtype, "h_in rows")
    assert_close(host(h_out[ri]), ref["h_out"], wl.dtype, "h_out rows")
    assert np.all(np.isfinite(host(out))) and np.all(np.isfinite(host(g["dx"])))
    rg = oracle.mlp_bwd(xv, *_wv(inp), inp.dout.v[rows], wl.r, wl.eps, dx_residual=inp.dout.v[rows])
    assert_close(host(g["dx"][ri]), rg["dx"], wl.dtype, "dx rows")
    for k in GRADS[1:]:
        assert np.all(np.isfinite(host(g[k]))), k


def test_mlp_degenerate_rows():
    """All-zero, constant and strongly scaled rows through the MLP, forward and
    backward, against the oracle on the same bf16 values."""
    from workloads import Tensor
    wl = MlpWorkload("mlp_degenerate", T=260, d=256, f=448, r=64, dtype="bf16", residual=True)
    _say("degenerate rows", wl)
    inp = make_mlp_inputs(wl, seed=6)
    xv = inp.x.v.copy()
    xv[0] = 0.0
    xv[100] = 2.0
    xv[101:104] *= 1e3
    xv[104:107] *= 1e-3
    xv[-1] = 0.0
    inp.x = Tensor(xv, wl.dtype)
    dims = _dims(wl)
    x = dev(inp.x)
    w = _weights(inp)
    out, h_in, h_out = rb.mlp_fwd(dims, x, *w, residual=x)
    dout = dev(inp.dout)
    g = rb.mlp_bwd(dims, x, *w, h_in, h_out, dout, dx_residual=dout)
    torch.cuda.synchronize()
    ref = oracle.mlp_fwd(inp.x.v, *_wv(inp), wl.r, wl.eps, residual=inp.x.v)
    assert_close(host(out), ref["out"], wl.dtype, "out")
    assert_close(host(h_in), ref["h_in"], wl.dtype, "h_in")
    rg = oracle.mlp_bwd(inp.x.v, *_wv(inp), inp.dout.v, wl.r, wl.eps, dx_residual=inp.dout.v)
    for k in GRADS:
        assert_close(host(g[k]), rg[k], wl.dtype, k)


def test_mlp_selection_case_exact():
    """x in {+-1}, gamma = 1, eps = 0, selection weights (the oracle's
    closed-form pin): every intermediate is a selection, so out equals
    SiLU(+-1) * (+-1) rounded once to the storage type; exact in bf16, within
    2 ulp of the device exp in fp32."""
    T, d, f, r = 300, 256, 320, 64
    x, gamma, A_in, B_g, B_u, A_o, B_o, *_ = mlp_selection_case(T, d, f, r, seed=3)
    ref = oracle.mlp_fwd(x, gamma, A_in, B_g, B_u, A_o, B_o, r, 0.0)["out"]
    for dtype, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        t = lambda a: torch.tensor(a, dtype=tdt, device="cuda").contiguous()
        dims = rb.make_mlp_dims(T, d, f, r, dtype, 0.0)
        out, _, _ = rb.mlp_fwd(dims, t(x), t(gamma), t(A_in), t(B_g), t(B_u), t(A_o), t(B_o))
        torch.cuda.synchronize()
        exp = torch.tensor(ref, dtype=tdt).double().numpy()
        tol = 0.0 if dtype == "bf16" else 2.5e-7
        assert np.max(np.abs(host(out) - exp)) <= tol, (dtype, np.max(np.abs(host(out) - exp)))
