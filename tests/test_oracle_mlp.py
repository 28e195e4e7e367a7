"""Pins of the per-projection low-rank SwiGLU MLP oracle (oracle/mlp.py), all on
the CPU: the element-by-element loops, torch autograd in float64 (an
independent implementation of every derivative, with torch's own RMSNorm and
SiLU), central differences of the loop version, the composition of the
already-pinned block oracle, and planted mistakes that these pins must catch."""
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

from util import mlp_selection_case

EPS = 1e-6


def _rand(rng, T, d, f, r):
    x = rng.standard_normal((T, d))
    gamma = 1 + 0.3 * rng.standard_normal(d)
    gamma[0] = -0.5                      # a negative scale, so |gamma| mistakes show
    A_in = rng.standard_normal((d, 2 * r)) / np.sqrt(d)
    B_g = rng.standard_normal((r, f)) / np.sqrt(r)
    B_u = rng.standard_normal((r, f)) / np.sqrt(r)
    A_o = rng.standard_normal((f, r)) / np.sqrt(f)
    B_o = rng.standard_normal((r, d)) / np.sqrt(r)
    return x, gamma, A_in, B_g, B_u, A_o, B_o


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _torch_grads(x, gamma, A_in, B_g, B_u, A_o, B_o, dout, r, residual=None):
    t = [torch.tensor(v, requires_grad=True) for v in (x, gamma, A_in, B_g, B_u, A_o, B_o)]
    tx, tg, tAi, tBg, tBu, tAo, tBo = t
    d = x.shape[1]
    xn = torch.nn.functional.rms_norm(tx, (d,), weight=tg, eps=EPS)
    h = xn @ tAi
    s = torch.nn.functional.silu(h[:, :r] @ tBg) * (h[:, r:] @ tBu)
    out = (s @ tAo) @ tBo
    if residual is not None:
        out = out + tx
    (out * torch.tensor(dout)).sum().backward()
    return out.detach().numpy(), [v.grad.numpy() for v in t]


@pytest.mark.parametrize("T,d,f,r", [(1, 4, 6, 1), (3, 8, 12, 2), (5, 6, 10, 3)])
@pytest.mark.parametrize("with_res", [False, True])
def test_mlp_forward_matches_loops(T, d, f, r, with_res):
    """The vectorised forward equals the element-by-element one."""
    rng = np.random.default_rng(T * 100 + d + f + r)
    x, gamma, A_in, B_g, B_u, A_o, B_o = _rand(rng, T, d, f, r)
    res = rng.standard_normal((T, d)) if with_res else None
    o = oracle.mlp_fwd(x, gamma, A_in, B_g, B_u, A_o, B_o, r, EPS, residual=res)
    lo = brute.mlp_fwd_loops(x.tolist(), gamma.tolist(), A_in.tolist(), B_g.tolist(), B_u.tolist(),
                             A_o.tolist(), B_o.tolist(), r, EPS, None if res is None else res.tolist())
    assert _rel(o["out"], lo) < 1e-13


@pytest.mark.parametrize("T,d,f,r", [(4, 8, 12, 2), (7, 16, 24, 4)])
def test_mlp_backward_matches_torch_autograd(T, d, f, r):
    """Every gradient against torch autograd in float64."""
    rng = np.random.default_rng(7 + T)
    x, gamma, A_in, B_g, B_u, A_o, B_o = _rand(rng, T, d, f, r)
    dout = rng.standard_normal((T, d))
    out, g = _torch_grads(x, gamma, A_in, B_g, B_u, A_o, B_o, dout, r)
    fw = oracle.mlp_fwd(x, gamma, A_in, B_g, B_u, A_o, B_o, r, EPS)
    bw = oracle.mlp_bwd(x, gamma, A_in, B_g, B_u, A_o, B_o, dout, r, EPS)
    assert _rel(fw["out"], out) < 1e-12
    for name, ref in zip(("dx", "dgamma", "dA_in", "dB_g", "dB_u", "dA_o", "dB_o"), g):
        assert _rel(bw[name], ref) < 1e-10, name


def test_mlp_residual_sublayer_matches_torch_autograd():
    """out = x + mlp(x): dx gains dout through the residual path."""
    T, d, f, r = 5, 8, 12, 2
    rng = np.random.default_rng(3)
    x, gamma, A_in, B_g, B_u, A_o, B_o = _rand(rng, T, d, f, r)
    dout = rng.standard_normal((T, d))
    out, g = _torch_grads(x, gamma, A_in, B_g, B_u, A_o, B_o, dout, r, residual=True)
    fw = oracle.mlp_fwd(x, gamma, A_in, B_g, B_u, A_o, B_o, r, EPS, residual=x)
    bw = oracle.mlp_bwd(x, gamma, A_in, B_g, B_u, A_o, B_o, dout, r, EPS, dx_residual=dout)
    assert _rel(fw["out"], out) < 1e-12
    assert _rel(bw["dx"], g[0]) < 1e-10
    assert _rel(bw["dA_o"], g[5]) < 1e-10


def test_mlp_backward_central_differences():
    """Entries of each gradient against central differences of the loop forward
    (loss = sum(out * dout))."""
    T, d, f, r = 3, 5, 7, 2
    rng = np.random.default_rng(11)
    args = list(_rand(rng, T, d, f, r))
    dout = rng.standard_normal((T, d))
    bw = oracle.mlp_bwd(*args, dout, r, EPS)

    def loss(a):
        o = brute.mlp_fwd_loops(*[v.tolist() for v in a], r, EPS)
        return float(np.sum(np.asarray(o) * dout))

    names = ("dx", "dgamma", "dA_in", "dB_g", "dB_u", "dA_o", "dB_o")
    h = 1e-6
    for k, name in enumerate(names):
        pick = rng.integers(0, args[k].size, size=3)
        for p in pick:
            idx = np.unravel_index(p, args[k].shape)
            plus = [v.copy() for v in args]
            minus = [v.copy() for v in args]
            plus[k][idx] += h
            minus[k][idx] -= h
            num = (loss(plus) - loss(minus)) / (2 * h)
            ana = np.asarray(bw[name])[idx]
            assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (name, idx, num, ana)


def test_mlp_input_layers_are_the_block():
    """The two input-side layers are the bottleneck block with identity between
    its factors, g = 2 and up-projections of width f; their backward is the
    block's backward for the upstream gradients (dgate, dup).  Ties this oracle
    to the separately pinned block oracle."""
    T, d, f, r = 6, 8, 20, 3
    rng = np.random.default_rng(5)
    x, gamma, A_in, B_g, B_u, A_o, B_o = _rand(rng, T, d, f, r)
    fw = oracle.mlp_fwd(x, gamma, A_in, B_g, B_u, A_o, B_o, r, EPS)
    blk = oracle.block_fwd(x, gamma, A_in, [B_g, B_u], r, 2, "identity", EPS)
    assert _rel(fw["gate"], blk["y"][0]) < 1e-14 and _rel(fw["up"], blk["y"][1]) < 1e-14
    assert _rel(fw["h_in"], blk["h"]) < 1e-14
    dout = rng.standard_normal((T, d))
    bw = oracle.mlp_bwd(x, gamma, A_in, B_g, B_u, A_o, B_o, dout, r, EPS)
    bb = oracle.block_bwd(x, gamma, A_in, [B_g, B_u], [bw["dgate"], bw["dup"]], r, 2, "identity", EPS)
    assert _rel(bw["dx"], bb["dx"]) < 1e-12 and _rel(bw["dgamma"], bb["dgamma"]) < 1e-12
    assert _rel(bw["dA_in"], bb["dA"]) < 1e-12
    assert _rel(bw["dB_g"], bb["dB"][0]) < 1e-12 and _rel(bw["dB_u"], bb["dB"][1]) < 1e-12


# ---------------------------------------------------------------- planted mistakes
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "mlp.py")

MUTATIONS = {
    "swiglu_swapped": ("s = _silu(gate) * up", "s = gate * _silu(up)"),
    "dgate_drops_up": ("dgate = ds * up * _dsilu(gate)", "dgate = ds * _dsilu(gate)"),
    "dup_no_silu": ("dup = ds * _silu(gate)", "dup = ds * gate"),
    "dA_o_uses_up": ("dA_o = s.T @ dh_out", "dA_o = up.T @ dh_out"),
    "dh_in_order": ("np.concatenate([dgate @ B_g.T, dup @ B_u.T], axis=1)",
                    "np.concatenate([dup @ B_u.T, dgate @ B_g.T], axis=1)"),
    "dB_u_from_gate_half": ("dB_u = h_in[:, r:].T @ dup", "dB_u = h_in[:, :r].T @ dup"),
    "residual_dropped": ("out = out + _f64(residual)", "out = out + 0.0 * _f64(residual)"),
    "dx_drops_correction": ("x * (rstd * rstd * dot / d)[:, None]", "0.0 * x"),
}


def _load_mutant(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert old in src, name
    src = src.replace(old, new, 1).replace("from .block import", "from oracle.block import")
    mod = types.ModuleType("oracle_mlp_mutant_" + name)
    exec(compile(src, SRC, "exec"), mod.__dict__)
    return mod


def _pins_hold(o) -> bool:
    """A compact run of the pins above on module `o`: loops (with a residual)
    and torch autograd (plain and residual)."""
    T, d, f, r = 4, 8, 12, 2
    rng = np.random.default_rng(2)
    x, gamma, A_in, B_g, B_u, A_o, B_o = _rand(rng, T, d, f, r)
    res = rng.standard_normal((T, d))
    fw = o.mlp_fwd(x, gamma, A_in, B_g, B_u, A_o, B_o, r, EPS, residual=res)
    lo = brute.mlp_fwd_loops(x.tolist(), gamma.tolist(), A_in.tolist(), B_g.tolist(), B_u.tolist(),
                             A_o.tolist(), B_o.tolist(), r, EPS, res.tolist())
    ok = _rel(fw["out"], lo) < 1e-12
    dout = rng.standard_normal((T, d))
    _, g = _torch_grads(x, gamma, A_in, B_g, B_u, A_o, B_o, dout, r)
    bw = o.mlp_bwd(x, gamma, A_in, B_g, B_u, A_o, B_o, dout, r, EPS)
    for name, ref in zip(("dx", "dgamma", "dA_in", "dB_g", "dB_u", "dA_o", "dB_o"), g):
        ok &= _rel(bw[name], ref) < 1e-10
    return bool(ok)


def test_unmutated_mlp_oracle_passes_compact_pins():
    from oracle import mlp
    assert _pins_hold(mlp)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mlp_pins_catch_planted_mistake(name):
    assert not _pins_hold(_load_mutant(name))


def test_mlp_selection_closed_form():
    """With selection weights every intermediate is a selection, so
    out[t, sel_o[k]] = SiLU(x[t, sel_g[k]]) * x[t, sel_u[k]], which takes the
    values e/(1+e), -e/(1+e), -1/(1+e), 1/(1+e) (SiLU(1) = e/(1+e), SiLU(-1) =
    -1/(1+e)); every other entry of out is 0."""
    import math
    T, d, f, r = 5, 8, 6, 3
    x, gamma, A_in, B_g, B_u, A_o, B_o, sel_g, sel_u, sel_o = mlp_selection_case(T, d, f, r)
    silu = {1.0: math.e / (1.0 + math.e), -1.0: -1.0 / (1.0 + math.e)}
    want = np.zeros((T, d))
    for t in range(T):
        for k in range(r):
            want[t, sel_o[k]] = silu[x[t, sel_g[k]]] * x[t, sel_u[k]]
    got = oracle.mlp_fwd(x, gamma, A_in, B_g, B_u, A_o, B_o, r, 0.0)["out"]
    assert np.max(np.abs(got - want)) <= 2e-16     # exp() may differ by an ulp
    assert set(np.round(np.abs(want[want != 0]), 12)) <= {round(math.e / (1 + math.e), 12),
                                                          round(1 / (1 + math.e), 12)}
