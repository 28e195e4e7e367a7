"""Pure-Python loop version of the block forward, for tiny shapes only (test
infrastructure).  Written element by element, without NumPy, so that it shares
no vectorised indexing with ``oracle.block``; the tests compare the two and
differentiate this one by central differences."""
from __future__ import annotations

import math
from typing import List


def silu(v: float) -> float:
    return v / (1.0 + math.exp(-v))


def block_fwd_loops(x: List[List[float]], gamma: List[float], A: List[List[float]],
                    B: List[List[List[float]]], r: int, g: int, act: str, eps: float,
                    D: int = 0, residual=None) -> List[List[List[float]]]:
    """y_i[t][j] for every up-projection i; `residual` (n_up lists [T][d]) is
    added to each output element when given."""
    T, d = len(x), len(x[0])
    D = D or d
    ys = []
    n_up = 1 if act == "swiglu" else g
    for i in range(n_up):
        ys.append([[0.0] * d for _ in range(T)])
    for t in range(T):
        acc = 0.0
        for j in range(d):
            acc += x[t][j] * x[t][j]
        rstd = 1.0 / math.sqrt(acc / D + eps)
        xn = [x[t][j] * rstd * gamma[j] for j in range(d)]
        h = []
        for c in range(g * r):
            s = 0.0
            for j in range(d):
                s += xn[j] * A[j][c]
            h.append(s)
        zs = []
        if act == "identity":
            zs = [h[i * r:(i + 1) * r] for i in range(g)]
        elif act == "silu":
            zs = [[silu(v) for v in h[i * r:(i + 1) * r]] for i in range(g)]
        elif act == "swiglu":
            zs = [[silu(h[k]) * h[r + k] for k in range(r)]]
        for i in range(n_up):
            for j in range(d):
                s = 0.0
                for k in range(r):
                    s += zs[i][k] * B[i][k][j]
                if residual is not None:
                    s += residual[i][t][j]
                ys[i][t][j] = s
    return ys


def mlp_fwd_loops(x: List[List[float]], gamma: List[float], A_in: List[List[float]],
                  B_g: List[List[float]], B_u: List[List[float]], A_o: List[List[float]],
                  B_o: List[List[float]], r: int, eps: float, residual=None) -> List[List[float]]:
    """out[t][j] of the per-projection low-rank SwiGLU MLP, element by element
    (`residual` [T][d] added when given)."""
    T, d = len(x), len(x[0])
    f = len(B_g[0])
    out = [[0.0] * d for _ in range(T)]
    for t in range(T):
        acc = 0.0
        for j in range(d):
            acc += x[t][j] * x[t][j]
        rstd = 1.0 / math.sqrt(acc / d + eps)
        xn = [x[t][j] * rstd * gamma[j] for j in range(d)]
        h = []
        for c in range(2 * r):
            v = 0.0
            for j in range(d):
                v += xn[j] * A_in[j][c]
            h.append(v)
        s = []
        for m in range(f):
            gv = 0.0
            uv = 0.0
            for k in range(r):
                gv += h[k] * B_g[k][m]
                uv += h[r + k] * B_u[k][m]
            s.append(silu(gv) * uv)
        ho = []
        for k in range(r):
            v = 0.0
            for m in range(f):
                v += s[m] * A_o[m][k]
            ho.append(v)
        for j in range(d):
            v = 0.0
            for k in range(r):
                v += ho[k] * B_o[k][j]
            if residual is not None:
                v += residual[t][j]
            out[t][j] = v
    return out
