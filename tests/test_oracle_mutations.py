"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks
that the pins notice each one: a dropped term, a wrong sign, a misplaced eps,
a swapped gate/up, a wrong width, a transposed operand."""
import importlib.util
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

from oracle import brute

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "block.py")

MUTATIONS = {
    "dx_drops_correction": ("x * (rstd * rstd * dot / D)[:, None]", "0.0 * x"),
    "dx_sign": ("gamma[None, :] * dxn - x", "gamma[None, :] * dxn + x"),
    "eps_outside_sqrt": ("1.0 / np.sqrt(ss / D + eps)\n    return ss, rstd",
                         "1.0 / np.sqrt(ss / D) + eps\n    return ss, rstd"),
    "mean_over_d_not_D": ("rstd = 1.0 / np.sqrt(ss / D + eps)\n    h = partial",
                          "rstd = 1.0 / np.sqrt(ss / partial.shape[0] + eps)\n    h = partial"),
    "dsilu_sign": ("s * (1.0 + v * (1.0 - s))", "s * (1.0 + v * (1.0 + s))"),
    "swiglu_swapped": ("return [_silu(hs[0]) * hs[1]]", "return [_silu(hs[1]) * hs[0]]"),
    "dgamma_no_rstd": ("np.sum(dxn * x * rstd[:, None], axis=0)", "np.sum(dxn * x, axis=0)"),
    "dA_uses_x": ("dA = xn.T @ dh", "dA = x.T @ dh"),
    "dh_up_wrong": ("dh[:, sl[1]] = dz[0] * _silu(hs[0])", "dh[:, sl[1]] = dz[0] * hs[0]"),
    "gamma_before_square": ("return x * rstd[:, None] * _f64(gamma)[None, :], ss, rstd",
                            "return x * rstd[:, None] * np.abs(_f64(gamma))[None, :], ss, rstd"),
    "branch_offset": ("return [slice(i * r, (i + 1) * r) for i in range(g)]",
                      "return [slice(i * r, (i + 1) * r) for i in range(g)][::-1]"),
    "residual_dropped": ("y = [yi + _f64(ri) for yi, ri in zip(y, residual)]",
                         "y = [yi + 0.0 * _f64(ri) for yi, ri in zip(y, residual)]"),
    "dx_residual_dropped": ("dx = dx + _f64(dx_residual)", "dx = dx - 0.0 * _f64(dx_residual)"),
}


def _load_mutant(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert old in src, name
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant_" + name)
    exec(compile(src, SRC, "exec"), mod.__dict__)
    return mod


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


def _pins_hold(o) -> bool:
    """A compact run of the pins: loops, torch autograd, library RMSNorm, the
    shard seam."""
    ok = True
    for act, g in (("silu", 2), ("swiglu", 2), ("identity", 3)):
        T, d, r, eps = 6, 16, 4, 1e-6
        rng = np.random.default_rng(1)
        n_up = 1 if act == "swiglu" else g
        x = rng.standard_normal((T, d)); gamma = 1 + 0.3 * rng.standard_normal(d)
        gamma[0] = -0.5
        A = rng.standard_normal((d, g * r)) / 4; B = [rng.standard_normal((r, d)) / 2 for _ in range(n_up)]
        dy = [rng.standard_normal((T, d)) for _ in range(n_up)]
        f = o.block_fwd(x, gamma, A, B, r, g, act, eps)
        yl = brute.block_fwd_loops(x.tolist(), gamma.tolist(), A.tolist(), [b.tolist() for b in B], r, g, act, eps)
        ok &= all(_rel(a, b) < 1e-12 for a, b in zip(f["y"], yl))
        tx = torch.tensor(x, requires_grad=True); tg = torch.tensor(gamma, requires_grad=True)
        tA = torch.tensor(A, requires_grad=True); tB = [torch.tensor(b, requires_grad=True) for b in B]
        xn = torch.nn.functional.rms_norm(tx, (d,), weight=tg, eps=eps)
        h = xn @ tA
        hs = [h[:, i * r:(i + 1) * r] for i in range(g)]
        z = hs if act == "identity" else ([torch.nn.functional.silu(v) for v in hs] if act == "silu"
                                          else [torch.nn.functional.silu(hs[0]) * hs[1]])
        ys = [zi @ Bi for zi, Bi in zip(z, tB)]
        sum((y * torch.tensor(t)).sum() for y, t in zip(ys, dy)).backward()
        bw = o.block_bwd(x, gamma, A, B, dy, r, g, act, eps)
        ok &= _rel(bw["dx"], tx.grad.numpy()) < 1e-10 and _rel(bw["dgamma"], tg.grad.numpy()) < 1e-10
        ok &= _rel(bw["dA"], tA.grad.numpy()) < 1e-10
        ok &= all(_rel(a, b.grad.numpy()) < 1e-10 for a, b in zip(bw["dB"], tB))
        # shard seam, 2 shards, normalising by the full width
        P, SS = 0, 0
        for s in range(2):
            c = slice(s * d // 2, (s + 1) * d // 2)
            p, ss = o.down_partial(x[:, c], gamma[c], A[c, :]); P = P + p; SS = SS + ss
        u = o.up_finish(P, SS, B, r, g, act, eps, d)
        ok &= all(_rel(a, b) < 1e-12 for a, b in zip(u["y"], f["y"]))
        y_lib = torch.nn.functional.rms_norm(torch.tensor(x), (d,), weight=torch.tensor(gamma), eps=eps)
        ok &= _rel(o.rmsnorm(x, gamma, eps)[0], y_lib.numpy()) < 1e-13
        # residual sublayer out = x + block(x) (first branch): loops and autograd
        res = [x] * n_up
        fr = o.block_fwd(x, gamma, A, B, r, g, act, eps, residual=res)
        ylr = brute.block_fwd_loops(x.tolist(), gamma.tolist(), A.tolist(), [b.tolist() for b in B], r, g, act, eps,
                                    residual=[x.tolist()] * n_up)
        ok &= all(_rel(a, b) < 1e-12 for a, b in zip(fr["y"], ylr))
        tx2 = torch.tensor(x, requires_grad=True)
        xn2 = torch.nn.functional.rms_norm(tx2, (d,), weight=torch.tensor(gamma), eps=eps)
        h2 = xn2 @ torch.tensor(A)
        hs2 = [h2[:, i * r:(i + 1) * r] for i in range(g)]
        z2 = hs2 if act == "identity" else ([torch.nn.functional.silu(v) for v in hs2] if act == "silu"
                                            else [torch.nn.functional.silu(hs2[0]) * hs2[1]])
        ((tx2 + z2[0] @ torch.tensor(B[0])) * torch.tensor(dy[0])).sum().backward()
        bwr = o.block_bwd(x, gamma, A, B, [dy[0]] + [0 * t for t in dy[1:]], r, g, act, eps, dx_residual=dy[0])
        ok &= _rel(bwr["dx"], tx2.grad.numpy()) < 1e-10
    return bool(ok)


def test_unmutated_oracle_passes_compact_pins():
    import oracle.block as ob
    assert _pins_hold(ob)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    assert not _pins_hold(_load_mutant(name)), f"planted mistake '{name}' went unnoticed"
