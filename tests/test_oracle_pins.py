"""Pins of the CPU oracle against things other than itself.

Each test names what it pins.  None of them compares the oracle with a retyped
copy of its own formula: the checks are brute-force loops, central
differences, torch's own RMSNorm / SiLU / autograd, closed forms, exact special
cases and invariants that the mathematics fixes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

ACTS = [("identity", 1), ("identity", 3), ("silu", 1), ("silu", 2), ("silu", 3), ("swiglu", 2)]


def _rand(rng, T, d, r, g, act, gstd=0.3):
    n_up = 1 if act == "swiglu" else g
    x = rng.standard_normal((T, d))
    gamma = 1.0 + gstd * rng.standard_normal(d)
    A = rng.standard_normal((d, g * r)) / math.sqrt(d)
    B = [rng.standard_normal((r, d)) / math.sqrt(r) for _ in range(n_up)]
    dy = [rng.standard_normal((T, d)) for _ in range(n_up)]
    return x, gamma, A, B, dy


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------- P1: brute force
@pytest.mark.parametrize("act,g", ACTS)
@pytest.mark.parametrize("T,d,r", [(1, 4, 1), (5, 8, 2), (8, 16, 4)])
def test_forward_matches_loops(act, g, T, d, r):
    """Oracle forward == element-by-element Python loops (indexing, branch
    layout of the concatenated A, which B goes with which branch)."""
    rng = np.random.default_rng(100 + T * 7 + d + r + g)
    x, gamma, A, B, _ = _rand(rng, T, d, r, g, act)
    f = oracle.block_fwd(x, gamma, A, B, r, g, act, 1e-6)
    yl = brute.block_fwd_loops(x.tolist(), gamma.tolist(), A.tolist(), [b.tolist() for b in B],
                               r, g, act, 1e-6)
    for yo, yb in zip(f["y"], yl):
        assert _rel(yo, yb) < 1e-12


def test_forward_loops_custom_norm_width():
    """Mean over D != d (a shard normalising by the unsharded width)."""
    rng = np.random.default_rng(7)
    x, gamma, A, B, _ = _rand(rng, 4, 8, 2, 1, "silu")
    f = oracle.block_fwd(x, gamma, A, B, 2, 1, "silu", 1e-6, D=32)
    yl = brute.block_fwd_loops(x.tolist(), gamma.tolist(), A.tolist(), [b.tolist() for b in B],
                               2, 1, "silu", 1e-6, D=32)
    assert _rel(f["y"][0], yl[0]) < 1e-12


# --------------------------------------------------------------------- P7: gradients
def _loss_loops(x, gamma, A, B, dy, r, g, act, eps, D=0):
    ys = brute.block_fwd_loops(x.tolist(), gamma.tolist(), A.tolist(), [b.tolist() for b in B],
                               r, g, act, eps, D)
    return sum(float(np.sum(np.asarray(y) * t)) for y, t in zip(ys, dy))


@pytest.mark.parametrize("act,g", [("identity", 2), ("silu", 1), ("silu", 3), ("swiglu", 2)])
def test_backward_central_differences(act, g):
    """Every gradient vs fp64 central differences of the loop forward, with the
    loss sum_i <y_i, dy_i>."""
    T, d, r, eps = 3, 6, 2, 1e-6
    rng = np.random.default_rng(11 + g)
    x, gamma, A, B, dy = _rand(rng, T, d, r, g, act)
    bw = oracle.block_bwd(x, gamma, A, B, dy, r, g, act, eps)
    step = 1e-6

    def fd(arr, setter):
        out = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += step
            m = arr.copy(); m[idx] -= step
            out[idx] = (setter(p) - setter(m)) / (2 * step)
        return out

    gx = fd(x, lambda v: _loss_loops(v, gamma, A, B, dy, r, g, act, eps))
    gg = fd(gamma, lambda v: _loss_loops(x, v, A, B, dy, r, g, act, eps))
    gA = fd(A, lambda v: _loss_loops(x, gamma, v, B, dy, r, g, act, eps))
    assert _rel(bw["dx"], gx) < 1e-6
    assert _rel(bw["dgamma"], gg) < 1e-6
    assert _rel(bw["dA"], gA) < 1e-6
    for i in range(len(B)):
        def with_Bi(v, i=i):
            Bs = list(B); Bs[i] = v
            return _loss_loops(x, gamma, A, Bs, dy, r, g, act, eps)
        assert _rel(bw["dB"][i], fd(B[i], with_Bi)) < 1e-6


def _torch_block(x, gamma, A, B, r, g, act, eps):
    """Independent forward in torch ops (library RMSNorm and SiLU)."""
    xn = torch.nn.functional.rms_norm(x, (x.shape[1],), weight=gamma, eps=eps)
    h = xn @ A
    hs = [h[:, i * r:(i + 1) * r] for i in range(g)]
    if act == "identity":
        z = hs
    elif act == "silu":
        z = [torch.nn.functional.silu(v) for v in hs]
    else:
        z = [torch.nn.functional.silu(hs[0]) * hs[1]]
    return [zi @ Bi for zi, Bi in zip(z, B)]


@pytest.mark.parametrize("act,g", ACTS)
def test_backward_matches_torch_autograd(act, g):
    """Forward and backward vs torch autograd (fp64, CPU) through torch's own
    rms_norm and silu."""
    T, d, r, eps = 24, 32, 8, 1e-6
    rng = np.random.default_rng(23 + g)
    x, gamma, A, B, dy = _rand(rng, T, d, r, g, act)
    tx = torch.tensor(x, requires_grad=True)
    tg = torch.tensor(gamma, requires_grad=True)
    tA = torch.tensor(A, requires_grad=True)
    tB = [torch.tensor(b, requires_grad=True) for b in B]
    ys = _torch_block(tx, tg, tA, tB, r, g, act, eps)
    loss = sum((y * torch.tensor(t)).sum() for y, t in zip(ys, dy))
    loss.backward()
    f = oracle.block_fwd(x, gamma, A, B, r, g, act, eps)
    bw = oracle.block_bwd(x, gamma, A, B, dy, r, g, act, eps)
    for yo, yt in zip(f["y"], ys):
        assert _rel(yo, yt.detach().numpy()) < 1e-12
    assert _rel(bw["dx"], tx.grad.numpy()) < 1e-12
    assert _rel(bw["dgamma"], tg.grad.numpy()) < 1e-12
    assert _rel(bw["dA"], tA.grad.numpy()) < 1e-12
    for dbo, tb in zip(bw["dB"], tB):
        assert _rel(dbo, tb.grad.numpy()) < 1e-12


def test_silu_and_derivative_vs_torch():
    """SiLU and SiLU' of the oracle vs torch.nn.functional.silu and its autograd."""
    v = np.linspace(-30, 30, 2001)
    tv = torch.tensor(v, requires_grad=True)
    s = torch.nn.functional.silu(tv)
    s.sum().backward()
    z = oracle.act_forward(v[:, None], "silu", 1, 1)[0][:, 0]
    dz = oracle.act_backward(v[:, None], [np.ones((v.size, 1))], "silu", 1, 1)[:, 0]
    assert np.max(np.abs(z - s.detach().numpy())) < 1e-13
    assert np.max(np.abs(dz - tv.grad.numpy())) < 1e-13


# --------------------------------------------------------------------- P2: closed form
@pytest.mark.parametrize("g", [1, 3])
def test_identity_closed_form(g):
    """sigma = identity: the block is one dense product, y_i = xn . (A_i B_i),
    and equally diag(rstd) . x . diag(gamma) . (A_i B_i)."""
    T, d, r, eps = 16, 32, 4, 1e-6
    rng = np.random.default_rng(3)
    x, gamma, A, B, _ = _rand(rng, T, d, r, g, "identity")
    f = oracle.block_fwd(x, gamma, A, B, r, g, "identity", eps)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    for i in range(g):
        W = A[:, i * r:(i + 1) * r] @ B[i]                   # d x d dense equivalent
        ref = (np.diag(rstd) @ x @ np.diag(gamma)) @ W
        assert _rel(f["y"][i], ref) < 1e-13


# --------------------------------------------------------------------- P3: exact case
def test_exact_selection_case_golden():
    """x in {+-1}, eps = 0, gamma = 1: rstd is exactly 1.  A_i selects input
    coordinates (one-hot columns) and B_i = A_i^T scatters them back, so y_i is
    sigma(x) on the selected coordinates and 0 elsewhere.  Values from the
    hand-written fixture tests/golden/exact_selection.json."""
    import json, os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "exact_selection.json")))
    x = np.array(fx["x"], dtype=np.float64)
    T, d = x.shape
    r, g = fx["r"], fx["g"]
    sel = fx["select"]
    A = np.zeros((d, g * r))
    for c, j in enumerate(sel):
        A[j, c] = 1.0
    B = [A[:, i * r:(i + 1) * r].T.copy() for i in range(g)]
    for act, key in (("identity", "y_identity"), ("silu", "y_silu")):
        f = oracle.block_fwd(x, np.ones(d), A, B, r, g, act, 0.0)
        for i in range(g):
            ref = np.array(fx[key][i])
            tol = 0.0 if act == "identity" else 2e-16   # exp() may differ by an ulp
            assert np.max(np.abs(f["y"][i] - ref)) <= tol, (act, i)


def test_silu_of_one_closed_form():
    """SiLU(1) = e/(1+e), SiLU(-1) = -1/(1+e)."""
    z = oracle.act_forward(np.array([[1.0, -1.0]]), "silu", 2, 1)[0][0]
    e = math.e
    assert abs(z[0] - e / (1 + e)) < 1e-16
    assert abs(z[1] + 1 / (1 + e)) < 1e-16


# --------------------------------------------------------------------- P4: scale invariance
@pytest.mark.parametrize("c", [0.25, 2.0, 32.0])
@pytest.mark.parametrize("act,g", [("silu", 3), ("swiglu", 2)])
def test_rmsnorm_scale_invariance(c, act, g):
    """RMSNorm(c x) == RMSNorm(x): exactly up to rounding with eps = 0.  With
    eps > 0 the row scale moves by (1 + eps/(c^2 ms))^(-1/2) - (1 + eps/ms)^(-1/2),
    at most eps/(2 c^2 ms) to first order (ms = mean square of the row); SiLU's
    slope stays below 1.1, so 2 eps/(c^2 min ms) bounds the relative change."""
    T, d, r = 8, 64, 8
    rng = np.random.default_rng(5)
    x, gamma, A, B, _ = _rand(rng, T, d, r, g, act)
    ms = np.min(np.mean(x * x, axis=1))
    for eps, tol in ((0.0, 1e-14), (1e-6, 2e-6 / (min(c, 1.0) ** 2 * ms))):
        y0 = oracle.block_fwd(x, gamma, A, B, r, g, act, eps)["y"]
        y1 = oracle.block_fwd(c * x, gamma, A, B, r, g, act, eps)["y"]
        for a, b in zip(y0, y1):
            assert _rel(b, a) < tol


# --------------------------------------------------------------------- P5: grouping
@pytest.mark.parametrize("act", ["identity", "silu"])
def test_grouped_equals_separate(act):
    """One grouped call (concatenated A, batched B) == g calls with g = 1."""
    T, d, r, g = 12, 32, 4, 3
    rng = np.random.default_rng(9)
    x, gamma, A, B, dy = _rand(rng, T, d, r, g, act)
    f = oracle.block_fwd(x, gamma, A, B, r, g, act, 1e-6)
    bw = oracle.block_bwd(x, gamma, A, B, dy, r, g, act, 1e-6)
    dx_sum = np.zeros_like(x)
    dg_sum = np.zeros_like(gamma)
    for i in range(g):
        Ai = A[:, i * r:(i + 1) * r]
        fi = oracle.block_fwd(x, gamma, Ai, [B[i]], r, 1, act, 1e-6)
        bi = oracle.block_bwd(x, gamma, Ai, [B[i]], [dy[i]], r, 1, act, 1e-6)
        assert _rel(f["y"][i], fi["y"][0]) < 1e-14
        assert _rel(bw["dA"][:, i * r:(i + 1) * r], bi["dA"]) < 1e-14
        assert _rel(bw["dB"][i], bi["dB"][0]) < 1e-14
        dx_sum += bi["dx"]
        dg_sum += bi["dgamma"]
    # the input gradients of the shared input add up over the branches
    assert _rel(bw["dx"], dx_sum) < 1e-13
    assert _rel(bw["dgamma"], dg_sum) < 1e-13


# --------------------------------------------------------------------- P6: online RMSNorm
def test_deferred_normalisation_and_library_rmsnorm():
    """Scaling the GEMM output by rstd == normalising first; the oracle RMSNorm
    == torch.nn.functional.rms_norm."""
    T, d, r, g, eps = 32, 64, 8, 2, 1e-6
    rng = np.random.default_rng(13)
    x, gamma, A, B, _ = _rand(rng, T, d, r, g, "silu")
    f = oracle.block_fwd(x, gamma, A, B, r, g, "silu", eps)
    ss = np.einsum("tj,tj->t", x, x)
    deferred = ((x * gamma[None, :]) @ A) / np.sqrt(ss / d + eps)[:, None]
    assert _rel(f["h"], deferred) < 1e-14
    y, _, _ = oracle.rmsnorm(x, gamma, eps)
    yt = torch.nn.functional.rms_norm(torch.tensor(x), (d,), weight=torch.tensor(gamma), eps=eps)
    assert _rel(y, yt.numpy()) < 1e-14


# --------------------------------------------------------------------- P7: Euler identities
@pytest.mark.parametrize("act,g", ACTS)
def test_euler_identities(act, g):
    """Homogeneity: y is 0-homogeneous in x when eps = 0, so <x_t, dx_t> = 0 per
    row; y_i is linear in B_i, so <B_i, dB_i> = <y_i, dy_i>; for sigma =
    identity y is linear in A and in gamma, so <A, dA> = <gamma, dgamma> =
    sum_i <y_i, dy_i>."""
    T, d, r = 10, 32, 4
    rng = np.random.default_rng(17)
    x, gamma, A, B, dy = _rand(rng, T, d, r, g, act)
    bw = oracle.block_bwd(x, gamma, A, B, dy, r, g, act, 0.0)
    f = oracle.block_fwd(x, gamma, A, B, r, g, act, 0.0)
    rowdot = np.sum(x * bw["dx"], axis=1)
    assert np.max(np.abs(rowdot)) < 1e-12 * np.max(np.abs(bw["dx"])) * d
    yd = [float(np.sum(y * t)) for y, t in zip(f["y"], dy)]
    for i in range(len(B)):
        assert abs(np.sum(B[i] * bw["dB"][i]) - yd[i]) < 1e-12 * max(1.0, abs(yd[i]))
    if act == "identity":
        tot = sum(yd)
        assert abs(np.sum(A * bw["dA"]) - tot) < 1e-11 * max(1.0, abs(tot))
        assert abs(np.sum(gamma * bw["dgamma"]) - tot) < 1e-11 * max(1.0, abs(tot))


# --------------------------------------------------------------------- P8: rank-r identities
@pytest.mark.parametrize("act,g", ACTS)
def test_rank_r_identities(act, g):
    """sum_k gamma_k dxn_tk x_tk = S_t / rstd_t with S_t = sum_c dh_tc h_tc, and
    dgamma_j = sum_c A_jc (xhat^T dh)_jc with xhat = diag(rstd) x: both RMSNorm
    backward reductions can be read off rank-r tensors."""
    T, d, r = 20, 48, 8
    rng = np.random.default_rng(19)
    x, gamma, A, B, dy = _rand(rng, T, d, r, g, act)
    bw = oracle.block_bwd(x, gamma, A, B, dy, r, g, act, 1e-6)
    lhs = np.sum(gamma[None, :] * bw["dxn"] * x, axis=1)
    S = np.sum(bw["dh"] * bw["h"], axis=1)
    assert _rel(lhs, S / bw["rstd"]) < 1e-13
    M = (x * bw["rstd"][:, None]).T @ bw["dh"]
    assert _rel(bw["dgamma"], np.sum(A * M, axis=1)) < 1e-13
    assert _rel(bw["dA"], gamma[:, None] * M) < 1e-13


# --------------------------------------------------------------------- P9: shard seam
@pytest.mark.parametrize("act,g", [("silu", 1), ("identity", 3), ("swiglu", 2)])
def test_btp_shard_decomposition(act, g):
    """Split d into TP = 4 shards: the partials and local sums of squares add up
    to the unsharded ones, and finishing the summed partial with the global
    width gives the unsharded block; each shard's y columns are the block's."""
    T, d, r, tp, eps = 16, 64, 8, 4, 1e-6
    rng = np.random.default_rng(29)
    x, gamma, A, B, _ = _rand(rng, T, d, r, g, act)
    f = oracle.block_fwd(x, gamma, A, B, r, g, act, eps)
    w = d // tp
    parts, sss = [], []
    for s in range(tp):
        cols = slice(s * w, (s + 1) * w)
        p, ss = oracle.down_partial(x[:, cols], gamma[cols], A[cols, :])
        parts.append(p); sss.append(ss)
    P, SS = sum(parts), sum(sss)
    assert _rel(P * (1.0 / np.sqrt(SS / d + eps))[:, None], f["h"]) < 1e-13
    for s in range(tp):
        cols = slice(s * w, (s + 1) * w)
        u = oracle.up_finish(P, SS, [b[:, cols] for b in B], r, g, act, eps, d)
        for i in range(len(B)):
            assert _rel(u["y"][i], f["y"][i][:, cols]) < 1e-13


# --------------------------------------------------------------------- residual variant
@pytest.mark.parametrize("act,g", [("identity", 3), ("silu", 1), ("swiglu", 2)])
def test_residual_forward_matches_loops(act, g):
    """y_i = residual_i + z_i . B_i: oracle vs the element-by-element loops."""
    T, d, r = 5, 8, 2
    rng = np.random.default_rng(31 + g)
    x, gamma, A, B, _ = _rand(rng, T, d, r, g, act)
    res = [rng.standard_normal((T, d)) for _ in B]
    f = oracle.block_fwd(x, gamma, A, B, r, g, act, 1e-6, residual=res)
    yl = brute.block_fwd_loops(x.tolist(), gamma.tolist(), A.tolist(), [b.tolist() for b in B], r, g, act, 1e-6,
                               residual=[t.tolist() for t in res])
    for yo, yb in zip(f["y"], yl):
        assert _rel(yo, yb) < 1e-12


@pytest.mark.parametrize("act,g", [("silu", 1), ("swiglu", 2)])
def test_residual_sublayer_matches_torch_autograd(act, g):
    """The pre-norm sublayer out = x + block(x) through torch autograd (torch's
    own rms_norm and silu): the oracle forward with residual_0 = x gives out, and
    its backward with dx_residual = dy_0 gives x.grad; the residual leaves dgamma,
    dA and dB as they are."""
    T, d, r, eps = 4, 12, 3, 1e-6
    rng = np.random.default_rng(41 + g)
    x, gamma, A, B, dy = _rand(rng, T, d, r, g, act)
    tx = torch.tensor(x, requires_grad=True)
    tg = torch.tensor(gamma, requires_grad=True)
    tA = torch.tensor(A, requires_grad=True)
    tB = [torch.tensor(b, requires_grad=True) for b in B]
    xn = torch.nn.functional.rms_norm(tx, (d,), weight=tg, eps=eps)
    h = xn @ tA
    hs = [h[:, i * r:(i + 1) * r] for i in range(g)]
    z = [torch.nn.functional.silu(hs[0])] if act == "silu" else [torch.nn.functional.silu(hs[0]) * hs[1]]
    out = tx + z[0] @ tB[0]
    (out * torch.tensor(dy[0])).sum().backward()
    f = oracle.block_fwd(x, gamma, A, B, r, g, act, eps, residual=[x])
    assert _rel(f["y"][0], out.detach().numpy()) < 1e-13
    bw = oracle.block_bwd(x, gamma, A, B, dy, r, g, act, eps, dx_residual=dy[0])
    assert _rel(bw["dx"], tx.grad.numpy()) < 1e-12
    assert _rel(bw["dgamma"], tg.grad.numpy()) < 1e-12
    assert _rel(bw["dA"], tA.grad.numpy()) < 1e-12
    assert _rel(bw["dB"][0], tB[0].grad.numpy()) < 1e-12


def test_residual_sublayer_central_differences():
    """dx of out = x + block(x) (residual_0 = x, dx_residual = dy_0) vs central
    differences of the loop forward."""
    T, d, r, eps, act, g = 3, 6, 2, 1e-6, "silu", 1
    rng = np.random.default_rng(53)
    x, gamma, A, B, dy = _rand(rng, T, d, r, g, act)

    def loss(xv):
        ys = brute.block_fwd_loops(xv.tolist(), gamma.tolist(), A.tolist(), [b.tolist() for b in B], r, g, act,
                                   eps, residual=[xv.tolist()])
        return float(np.sum(np.asarray(ys[0]) * dy[0]))

    fd = np.zeros_like(x)
    step = 1e-6
    for idx in np.ndindex(x.shape):
        p = x.copy(); p[idx] += step
        m = x.copy(); m[idx] -= step
        fd[idx] = (loss(p) - loss(m)) / (2 * step)
    bw = oracle.block_bwd(x, gamma, A, B, dy, r, g, act, eps, dx_residual=dy[0])
    assert _rel(bw["dx"], fd) < 1e-6


# --------------------------------------------------------------------- working precision
def test_working_precision_float32():
    """The same oracle code in float32 (the CPU speed baseline's second leg)
    returns float32 arrays within float32 rounding of the float64 result, and
    the default stays float64 afterwards."""
    rng = np.random.default_rng(61)
    x, gamma, A, B, dy = _rand(rng, 64, 128, 16, 3, "silu")
    ref = oracle.block_bwd(x, gamma, A, B, dy, 16, 3, "silu", 1e-6)
    with oracle.working_precision(np.float32):
        f32 = oracle.block_bwd(x, gamma, A, B, dy, 16, 3, "silu", 1e-6)
    assert f32["dx"].dtype == np.float32 and f32["dA"].dtype == np.float32
    for k in ("dx", "dgamma", "dA"):
        assert _rel(f32[k], ref[k]) < 1e-5, k
    assert oracle.block_fwd(x, gamma, A, B, 16, 3, "silu", 1e-6)["y"][0].dtype == np.float64
