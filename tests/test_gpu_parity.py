"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases run the oracle on everything and span several 256 x 256 tiles with
ragged tails in T and in the rank dimension; full-size cases use the shapes and
launch configuration the benchmark times and compare sampled rows (rows are
independent in the forward and in dx) and, where affordable, whole gradients.
Tolerances: bf16 max|e| <= 1e-2 max|ref| and ||e||_F <= 5e-3 ||ref||_F; fp32 1e-5.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import rank_bottleneck_amd as rb
from workloads import WORKLOADS, Workload, make_inputs

from util import assert_close, dev, host

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-parity]", *a, file=sys.stderr, flush=True)


def _dims(wl: Workload, T=None):
    return rb.make_dims(wl.T if T is None else T, wl.d, wl.r, wl.g, wl.act, wl.dtype, wl.eps, wl.d_norm)


def _run_fwd(wl, inp, save_h=True):
    dims = _dims(wl, inp.x.shape[0])
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    y, h = rb.fwd(dims, x, gamma, A, B, save_h=save_h)
    torch.cuda.synchronize()
    return dims, (x, gamma, A, B), y, h


SMALL = [
    Workload("tiny_f32_silu", 128, 256, 64, 1, "silu", "f32"),
    Workload("f32_ragged", 300, 320, 128, 3, "silu", "f32"),
    Workload("f32_swiglu", 200, 256, 192, 2, "swiglu", "f32"),
    Workload("bf16_identity", 700, 512, 320, 3, "identity", "bf16"),
    Workload("bf16_silu", 555, 768, 192, 3, "silu", "bf16"),
    Workload("bf16_swiglu", 777, 1024, 256, 2, "swiglu", "bf16"),
    Workload("bf16_g1_r64", 1000, 512, 64, 1, "silu", "bf16"),
    Workload("bf16_dnorm", 333, 384, 128, 2, "silu", "bf16", d_norm=1536),
    # g*r <= 256 with few row tiles: the split-K small-rank forward
    Workload("bf16_swiglu_r64", 640, 256, 64, 2, "swiglu", "bf16"),
    Workload("bf16_identity_r128", 513, 320, 128, 1, "identity", "bf16"),
    # g = 1, r <= 256: the one-kernel small-rank forward (ragged T, a half-empty
    # last column tile, a normalization width other than d)
    Workload("bf16_g1_r256", 257, 448, 256, 1, "silu", "bf16"),
    Workload("bf16_g1_r128_dnorm", 130, 192, 128, 1, "silu", "bf16", d_norm=768),
    # SwiGLU's gate/up pair at small rank: the one-kernel forward as well
    Workload("bf16_swiglu_r128_small", 333, 320, 128, 2, "swiglu", "bf16"),
    # grouped branches at small g*r in the one-kernel forward (g*r = 192, 256)
    Workload("bf16_g3_r64", 519, 320, 64, 3, "silu", "bf16"),
    Workload("bf16_g4_r64", 200, 256, 64, 4, "identity", "bf16"),
    # a small g*r that the one-kernel forward does not take (r = 192): the
    # split-K down-projection, the finish kernel and the short-K up-projection
    Workload("bf16_g1_r192_split", 600, 384, 192, 1, "silu", "bf16"),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_block_forward_backward_small(wl):
    _say("small", wl)
    inp = make_inputs(wl, seed=1)
    dims, (x, gamma, A, B), y, h = _run_fwd(wl, inp)
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(h), ref["h"], wl.dtype, "h")
    for i, yi in enumerate(y):
        assert_close(host(yi), ref["y"][i], wl.dtype, f"y{i}")
    dy = [dev(t) for t in inp.dy]
    g = rb.bwd(dims, x, gamma, A, B, h, dy)
    torch.cuda.synchronize()
    rb_ = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], [t.v for t in inp.dy],
                           wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(g["dx"]), rb_["dx"], wl.dtype, "dx")
    assert_close(host(g["dgamma"]), rb_["dgamma"], wl.dtype, "dgamma")
    assert_close(host(g["dA"]), rb_["dA"], wl.dtype, "dA")
    for i in range(len(B)):
        assert_close(host(g["dB"][i]), rb_["dB"][i], wl.dtype, f"dB{i}")


# The small cases above have fewer 256 x 256 down tiles than CUs, so their
# down-projection runs on 64-row tiles.  These shapes (ragged T, 396 and 264
# tiles) run the 256 x 256 tiles, with a full and a nearly empty last round.
@pytest.mark.parametrize("wl", [Workload("bf16_main_tiles", 8269, 128, 1536, 2, "silu", "bf16"),
                                Workload("bf16_main_tiles_tail", 8269, 128, 1024, 2, "silu", "bf16")],
                         ids=lambda w: w.name)
def test_forward_down_tile_configs_ragged(wl):
    _say("tile config", wl)
    inp = make_inputs(wl, seed=2, with_dy=False)
    _, _, y, h = _run_fwd(wl, inp)
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(h), ref["h"], wl.dtype, "h")
    for i, yi in enumerate(y):
        assert_close(host(yi), ref["y"][i], wl.dtype, f"y{i}")


def test_backward_256_tiles_ragged():
    """More than one round of 256 x 256 tiles in down and dz (260, ragged T) at a
    size the oracle takes whole; every gradient compared in full."""
    wl = Workload("bf16_bwd_tiles", 16461, 128, 1024, 1, "silu", "bf16")
    _say("256 tiles bwd", wl)
    inp = make_inputs(wl, seed=3)
    dims, (x, gamma, A, B), y, h = _run_fwd(wl, inp)
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(h), ref["h"], wl.dtype, "h")
    assert_close(host(y[0]), ref["y"][0], wl.dtype, "y0")
    g = rb.bwd(dims, x, gamma, A, B, h, [dev(t) for t in inp.dy])
    torch.cuda.synchronize()
    rb_ = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], [t.v for t in inp.dy],
                           wl.r, wl.g, wl.act, wl.eps, wl.D)
    for k in ("dx", "dgamma", "dA"):
        assert_close(host(g[k]), rb_[k], wl.dtype, k)
    assert_close(host(g["dB"][0]), rb_["dB"][0], wl.dtype, "dB0")


@pytest.mark.parametrize("wl", [SMALL[1], SMALL[2], SMALL[4], SMALL[5], SMALL[6], SMALL[7], SMALL[8], SMALL[13],
                                SMALL[15]], ids=lambda w: w.name)
def test_saved_rstd(wl):
    """The forward's rstd output (every forward path: 256 x 256 tiles, SwiGLU's
    gate/up tiles, fp32, the one-kernel forward alone and with grouped branches,
    the split-K small-rank path, a normalisation width other than d) against the
    oracle's statistic, and the backward fed that saved rstd."""
    _say("saved rstd", wl)
    inp = make_inputs(wl, seed=7)
    dims = _dims(wl)
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    rstd = torch.full((wl.T,), float("nan"), dtype=torch.float32, device="cuda")
    y, h = rb.fwd(dims, x, gamma, A, B, rstd=rstd)
    torch.cuda.synchronize()
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(rstd), ref["rstd"], "f32", "rstd")
    assert_close(host(h), ref["h"], wl.dtype, "h")
    g = rb.bwd(dims, x, gamma, A, B, h, [dev(t) for t in inp.dy], rstd=rstd)
    torch.cuda.synchronize()
    rb_ = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], [t.v for t in inp.dy],
                           wl.r, wl.g, wl.act, wl.eps, wl.D)
    for k in ("dx", "dgamma", "dA"):
        assert_close(host(g[k]), rb_[k], wl.dtype, k)
    for i in range(len(B)):
        assert_close(host(g["dB"][i]), rb_["dB"][i], wl.dtype, f"dB{i}")


@pytest.mark.parametrize("wl", [Workload("bf16_sk_interleave3", 2048, 2048, 512, 3, "identity", "bf16"),
                                Workload("bf16_sk_interleave2", 2048, 1024, 1024, 1, "silu", "bf16")],
                         ids=lambda w: w.name)
def test_backward_streamk_interleaved(wl):
    """Stream-K weight gradients whose tile sequence is interleaved: 96 tiles of 32
    k steps on 256 work-groups (3 tiles between work-groups of one XCD), and 32
    tiles of 32 k steps on 128 (2 tiles); every gradient compared in full."""
    _say("stream-K interleave bwd", wl)
    inp = make_inputs(wl, seed=5)
    dims, (x, gamma, A, B), y, h = _run_fwd(wl, inp)
    g = rb.bwd(dims, x, gamma, A, B, h, [dev(t) for t in inp.dy])
    torch.cuda.synchronize()
    ref = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], [t.v for t in inp.dy],
                           wl.r, wl.g, wl.act, wl.eps, wl.D)
    for k in ("dx", "dgamma", "dA"):
        assert_close(host(g[k]), ref[k], wl.dtype, k)
    for i in range(len(B)):
        assert_close(host(g["dB"][i]), ref["dB"][i], wl.dtype, f"dB{i}")


@pytest.mark.parametrize("wl", [SMALL[1], SMALL[4], SMALL[5], SMALL[8], SMALL[9], SMALL[10]], ids=lambda w: w.name)
def test_inference_forward_without_checkpoint(wl):
    inp = make_inputs(wl, seed=2, with_dy=False)
    _, _, y, h = _run_fwd(wl, inp, save_h=False)
    assert h is None
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps, wl.D)
    for i, yi in enumerate(y):
        assert_close(host(yi), ref["y"][i], wl.dtype, f"y{i}")


@pytest.mark.parametrize("T,d,r,act", [(1, 64, 64, "silu"), (63, 128, 128, "identity"), (65, 192, 256, "silu"),
                                        (64, 64, 256, "identity"), (129, 128, 64, "silu"), (1, 64, 64, "swiglu"),
                                        (97, 192, 128, "swiglu")])
def test_fused_forward_edges(T, d, r, act):
    """The one-kernel small-rank forward at its edges: a single token, a partly
    filled last row block, widths where every column tile past the first is
    padding (d = 64, 128) or half filled (d = 192), with and without the
    checkpoint."""
    g = 2 if act == "swiglu" else 1
    wl = Workload("fused_edge", T, d, r, g, act, "bf16")
    _say("fused edge", wl)
    inp = make_inputs(wl, seed=6, with_dy=False)
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], r, g, act, wl.eps, wl.D)
    for save_h in (True, False):
        _, _, y, h = _run_fwd(wl, inp, save_h=save_h)
        if save_h:
            assert_close(host(h), ref["h"], "bf16", "h")
        assert_close(host(y[0]), ref["y"][0], "bf16", "y0")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rmsnorm_online(dtype):
    wl = Workload("rms", 1111, 4096, 64, 1, "silu", dtype)
    inp = make_inputs(wl, seed=3, with_dy=False)
    dims = _dims(wl)
    x, gamma = dev(inp.x), dev(inp.gamma)
    y = torch.empty_like(x)
    ss = torch.empty(wl.T, dtype=torch.float32, device="cuda")
    rs = torch.empty_like(ss)
    rb.rmsnorm_online(dims, x, gamma, y, ss, rs)
    torch.cuda.synchronize()
    ry, rss, rrs = oracle.rmsnorm(inp.x.v, inp.gamma.v, wl.eps)
    assert_close(host(ss), rss, "f32", "sumsq")
    assert_close(host(rs), rrs, "f32", "rstd")
    assert_close(host(y), ry, dtype, "y")


@pytest.mark.parametrize("act,g", [("silu", 1), ("identity", 3), ("swiglu", 2)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shard_seam_small(act, g, dtype):
    """Partial + finish on one shard equals the oracle's seam; summing four
    shards' partials and finishing equals the unsharded block."""
    T, dl, r, tp = 500, 256, 128, 4
    wl = Workload("seam", T, dl * tp, r, g, act, dtype)
    inp = make_inputs(wl, seed=4, with_dy=False)
    full = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], r, g, act, wl.eps)
    parts, sss = [], []
    for s in range(tp):
        c = slice(s * dl, (s + 1) * dl)
        dims = rb.make_dims(T, dl, r, g, act, dtype, wl.eps, d_norm=dl * tp)
        x = dev(inp.x.store[:, c].copy() if dtype == "bf16" else inp.x.store[:, c])
        gm = dev(inp.gamma.store[c].copy())
        As = dev(inp.A.store[c, :].copy())
        p, ss = rb.down_partial(dims, x, gm, As)
        torch.cuda.synchronize()
        rp, rss = oracle.down_partial(inp.x.v[:, c], inp.gamma.v[c], inp.A.v[c, :])
        assert_close(host(p), rp, dtype, "partial")
        assert_close(host(ss), rss, "f32", "sumsq")
        parts.append(p)
        sss.append(ss)
    P = torch.stack(parts).sum(0).contiguous()   # stands in for the all-reduce
    SS = torch.stack(sss).sum(0).contiguous()
    # the finish step on its own: both sides take the oracle's summed partials
    # (rounded once to the fp32 the entry point takes)
    rps = [oracle.down_partial(inp.x.v[:, slice(s * dl, (s + 1) * dl)], inp.gamma.v[s * dl:(s + 1) * dl],
                               inp.A.v[s * dl:(s + 1) * dl, :]) for s in range(tp)]
    P_or = np.float32(sum(p for p, _ in rps))
    SS_or = np.float32(sum(q for _, q in rps))
    for s in range(tp):
        c = slice(s * dl, (s + 1) * dl)
        dims = rb.make_dims(T, dl, r, g, act, dtype, wl.eps, d_norm=dl * tp)
        Bs = [dev(b.store[:, c].copy()) for b in inp.B]
        y, h = rb.up_finish(dims, dev(P_or), dev(SS_or), Bs)
        torch.cuda.synchronize()
        ref = oracle.up_finish(P_or.astype(np.float64), SS_or.astype(np.float64), [b.v[:, c] for b in inp.B], r, g,
                               act, wl.eps, dl * tp)
        assert_close(host(h), ref["h"], dtype, "h")
        for i, yi in enumerate(y):
            assert_close(host(yi), ref["y"][i], dtype, "y (seam)")
        # the whole seam on the GPU (its partials summed in place of the
        # all-reduce) against the unsharded block
        y2, _ = rb.up_finish(dims, P, SS, Bs)
        torch.cuda.synchronize()
        for i, yi in enumerate(y2):
            assert_close(host(yi), full["y"][i][:, c], dtype, "y (vs unsharded)")


@pytest.mark.parametrize("T,d,r,g", [(300, 256, 64, 2), (300, 512, 256, 1)])
def test_exact_selection_case_bitwise(T, d, r, g):
    """x in {+-1}, eps = 0, gamma = 1, one-hot A, B = A^T: the GPU output is
    exact (identity) and equals the rounded SiLU(+-1) (SiLU), in fp32 and bf16
    (g = 1 in bf16 runs the one-kernel small-rank forward)."""
    rng = np.random.default_rng(0)
    x = np.where(rng.random((T, d)) < 0.5, -1.0, 1.0)
    sel = rng.permutation(d)[: g * r]
    A = np.zeros((d, g * r))
    A[sel, np.arange(g * r)] = 1.0
    B = [A[:, i * r:(i + 1) * r].T.copy() for i in range(g)]
    for dtype, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        for act in ("identity", "silu"):
            dims = rb.make_dims(T, d, r, g, act, dtype, 0.0)
            t = lambda a: torch.tensor(a, dtype=tdt, device="cuda").contiguous()
            y, _ = rb.fwd(dims, t(x), t(np.ones(d)), t(A), [t(b) for b in B])
            torch.cuda.synchronize()
            ref = oracle.block_fwd(x, np.ones(d), A, B, r, g, act, 0.0)
            for i in range(g):
                exp = torch.tensor(ref["y"][i], dtype=tdt).double().numpy()  # rounded once to the storage type
                got = host(y[i])
                if act == "identity":
                    assert np.array_equal(got, exp), (dtype, act, i)
                else:
                    # SiLU(+-1) through the device exp: within 2 ulp of fp32, exact after bf16 rounding
                    tol = 0.0 if dtype == "bf16" else 2.5e-7
                    assert np.max(np.abs(got - exp)) <= tol, (dtype, act, i, np.max(np.abs(got - exp)))


@pytest.mark.parametrize("wl", [SMALL[4], Workload("bf16_g3_r64_rerun", 300, 256, 64, 3, "silu", "bf16")],
                         ids=lambda w: w.name)
def test_deterministic_rerun(wl):
    """Bitwise-equal outputs on a second call (the grouped GEMM path, and the
    one-kernel forward with its fixed partial-sum order)."""
    inp = make_inputs(wl, seed=5)
    dims, (x, gamma, A, B), y1, h1 = _run_fwd(wl, inp)
    y2, h2 = rb.fwd(dims, x, gamma, A, B)
    dy = [dev(t) for t in inp.dy]
    g1 = rb.bwd(dims, x, gamma, A, B, h1, dy)
    g2 = rb.bwd(dims, x, gamma, A, B, h1, dy)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2) and all(torch.equal(a, b) for a, b in zip(y1, y2))
    for k in ("dx", "dgamma", "dA"):
        assert torch.equal(g1[k], g2[k]), k
    assert all(torch.equal(a, b) for a, b in zip(g1["dB"], g2["dB"]))


def test_empty_batch():
    """T = 0: no rows to produce; the weight gradients are sums over no tokens, so zero."""
    wl = Workload("empty", 0, 256, 64, 3, "silu", "bf16")
    dims = _dims(wl)
    dt = torch.bfloat16
    x = torch.empty((0, 256), dtype=dt, device="cuda")
    gamma = torch.ones(256, dtype=dt, device="cuda")
    A = torch.randn(256, 192, device="cuda").to(dt)
    B = [torch.randn(64, 256, device="cuda").to(dt) for _ in range(3)]
    rstd = torch.empty(0, dtype=torch.float32, device="cuda")
    y, h = rb.fwd(dims, x, gamma, A, B, rstd=rstd)
    g = rb.bwd(dims, x, gamma, A, B, h, [torch.empty((0, 256), dtype=dt, device="cuda")] * 3, rstd=rstd)
    torch.cuda.synchronize()
    assert y[0].shape == (0, 256) and h.shape == (0, 192)
    assert float(g["dA"].abs().max()) == 0.0 and float(g["dgamma"].abs().max()) == 0.0
    assert all(float(t.abs().max()) == 0.0 for t in g["dB"])


def test_status_on_bad_call_launches_nothing():
    dims = rb.make_dims(64, 100, 64, 1)
    x = torch.zeros((64, 100), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rb.LrError) as e:
        rb.lr_block_fwd(dims, x, x, x, [x], [x], None, x)
    assert e.value.status == rb.LR_EUNSUPPORTED


# ------------------------------------------------------------------ full-size shapes
FULL_FWD = ["qkv_identity", "swiglu_mlp", "qkv_silu_ckpt", "small_r64", "small_r128", "small_r256",
            "small_swiglu_r64", "small_swiglu_r128", "vanilla_tp_shard"]


def _sample_rows(T, n=1024, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.choice(T, n - 8, replace=False), np.arange(T - 8, T)]))
    return rows


@pytest.mark.parametrize("name", FULL_FWD)
def test_full_size_forward_sampled_rows(name):
    wl = WORKLOADS[name]
    _say("full fwd", wl)
    inp = make_inputs(wl, seed=0, with_dy=False)
    dims = _dims(wl)
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    rstd = torch.full((wl.T,), float("nan"), dtype=torch.float32, device="cuda")
    y, h = rb.fwd(dims, x, gamma, A, B, rstd=rstd)
    torch.cuda.synchronize()
    rows = _sample_rows(wl.T)
    ref = oracle.block_fwd(inp.x.v[rows], inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act,
                           wl.eps, wl.D)
    assert_close(host(rstd[torch.as_tensor(rows, device="cuda")]), ref["rstd"], "f32", "rstd rows")
    assert np.all(np.isfinite(host(rstd))), "rstd: a row was not written"
    assert_close(host(h[torch.as_tensor(rows, device="cuda")]), ref["h"], wl.dtype, "h rows")
    for i, yi in enumerate(y):
        assert_close(host(yi[torch.as_tensor(rows, device="cuda")]), ref["y"][i], wl.dtype, f"y{i} rows")


def test_full_size_btp_shard_seam():
    wl = WORKLOADS["btp_shard"]
    _say("full seam", wl)
    inp = make_inputs(wl, seed=0, with_dy=False)
    dims = _dims(wl)
    p, ss = rb.down_partial(dims, dev(inp.x), dev(inp.gamma), dev(inp.A))
    y, h = rb.up_finish(dims, p, ss, [dev(b) for b in inp.B])
    torch.cuda.synchronize()
    rows = _sample_rows(wl.T)
    rp, rss = oracle.down_partial(inp.x.v[rows], inp.gamma.v, inp.A.v)
    ri = torch.as_tensor(rows, device="cuda")
    assert_close(host(p[ri]), rp, wl.dtype, "partial rows")
    assert_close(host(ss[ri]), rss, "f32", "sumsq rows")
    ref = oracle.up_finish(rp, rss, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(y[0][ri]), ref["y"][0], wl.dtype, "y rows")


@pytest.mark.parametrize("name", ["qkv_silu_ckpt", "swiglu_mlp", "qkv_identity"])
def test_full_size_backward(name):
    """Whole-tensor comparison of every gradient at the full shape (the oracle's
    float64 products over all T take seconds on the host)."""
    wl = WORKLOADS[name]
    _say("full bwd", wl)
    inp = make_inputs(wl, seed=0)
    dims = _dims(wl)
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    # as the benchmark runs the step: rstd kept from the forward
    rstd = torch.full((wl.T,), float("nan"), dtype=torch.float32, device="cuda")
    y, h = rb.fwd(dims, x, gamma, A, B, rstd=rstd)
    del y
    g = rb.bwd(dims, x, gamma, A, B, h, [dev(t) for t in inp.dy], rstd=rstd)
    torch.cuda.synchronize()
    ref = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], [t.v for t in inp.dy],
                           wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(rstd), ref["rstd"], "f32", "rstd")
    assert_close(host(g["dx"]), ref["dx"], wl.dtype, "dx")
    assert_close(host(g["dgamma"]), ref["dgamma"], wl.dtype, "dgamma")
    assert_close(host(g["dA"]), ref["dA"], wl.dtype, "dA")
    for i in range(len(B)):
        assert_close(host(g["dB"][i]), ref["dB"][i], wl.dtype, f"dB{i}")


# ------------------------------------------------------------------ grouped branches up to MAX_G
@pytest.mark.parametrize("wl", [
    # g = 8 at r = 64: eight concatenated down-projections and eight batched up-projections
    Workload("bf16_g8_r64", 700, 512, 64, 8, "silu", "bf16"),
    # g = 5 at r = 1024: 5 x 8 = 40 S' row partials, more than the 32 the dx
    # kernel loads ahead of its epilogue, so its tail loop runs
    Workload("bf16_g5_r1024", 600, 256, 1024, 5, "silu", "bf16"),
    Workload("f32_g8_r64", 130, 256, 64, 8, "identity", "f32"),
], ids=lambda w: w.name)
def test_many_branches_whole_gradients(wl):
    _say("many branches", wl)
    inp = make_inputs(wl, seed=9)
    dims = _dims(wl)
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    for keep_rstd in (False, True):
        rstd = torch.full((wl.T,), float("nan"), dtype=torch.float32, device="cuda") if keep_rstd else None
        y, h = rb.fwd(dims, x, gamma, A, B, rstd=rstd)
        g = rb.bwd(dims, x, gamma, A, B, h, [dev(t) for t in inp.dy], rstd=rstd)
        torch.cuda.synchronize()
        ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps)
        assert_close(host(h), ref["h"], wl.dtype, "h")
        for i, yi in enumerate(y):
            assert_close(host(yi), ref["y"][i], wl.dtype, f"y{i}")
        rb_ = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], [t.v for t in inp.dy],
                               wl.r, wl.g, wl.act, wl.eps)
        for k in ("dx", "dgamma", "dA"):
            assert_close(host(g[k]), rb_[k], wl.dtype, k)
        for i in range(len(B)):
            assert_close(host(g["dB"][i]), rb_["dB"][i], wl.dtype, f"dB{i}")


# ------------------------------------------------------------------ residual variant
RESIDUAL = [
    # the GEMM path: SwiGLU sublayer out = x + block(x), r = 1024
    Workload("res_swiglu_r1024", 700, 1024, 1024, 2, "swiglu", "bf16"),
    # per-branch residuals with three up-projections
    Workload("res_identity_g3", 555, 512, 320, 3, "identity", "bf16"),
    # small rank: shapes the one-kernel forward takes without a residual
    Workload("res_swiglu_r64", 1000, 512, 64, 2, "swiglu", "bf16"),
    Workload("res_silu_r256", 333, 448, 256, 1, "silu", "bf16"),
    Workload("res_f32", 300, 320, 128, 1, "silu", "f32"),
]


@pytest.mark.parametrize("wl", RESIDUAL, ids=lambda w: w.name)
def test_residual_forward_backward(wl):
    """lr_block_fwd_residual / lr_block_bwd_residual against the oracle's
    residual variant: the first branch's residual is x (the sublayer
    out = x + block(x), whose dx gains dy_0), the others seeded draws."""
    _say("residual", wl)
    inp = make_inputs(wl, seed=12)
    rng = np.random.default_rng(13)
    extra = [workloads_tensor(rng.standard_normal((wl.T, wl.d)), wl.dtype) for _ in range(wl.n_up - 1)]
    res_h = [inp.x] + extra
    dims = _dims(wl)
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    res = [x] + [dev(t) for t in extra]
    rstd = torch.empty(wl.T, dtype=torch.float32, device="cuda")
    y, h = rb.fwd(dims, x, gamma, A, B, rstd=rstd, residual=res)
    dy = [dev(t) for t in inp.dy]
    g = rb.bwd(dims, x, gamma, A, B, h, dy, rstd=rstd, dx_residual=dy[0])
    torch.cuda.synchronize()
    Bv = [b.v for b in inp.B]
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, Bv, wl.r, wl.g, wl.act, wl.eps, wl.D,
                           residual=[t.v for t in res_h])
    assert_close(host(h), ref["h"], wl.dtype, "h")
    for i, yi in enumerate(y):
        assert_close(host(yi), ref["y"][i], wl.dtype, f"y{i}")
    rbw = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, Bv, [t.v for t in inp.dy], wl.r, wl.g, wl.act, wl.eps,
                           wl.D, dx_residual=inp.dy[0].v)
    for k in ("dx", "dgamma", "dA"):
        assert_close(host(g[k]), rbw[k], wl.dtype, k)
    for i in range(len(B)):
        assert_close(host(g["dB"][i]), rbw["dB"][i], wl.dtype, f"dB{i}")


@pytest.mark.parametrize("wl", [RESIDUAL[0], RESIDUAL[2]], ids=lambda w: w.name)
def test_residual_in_place(wl):
    """The residual accumulated in place (y_i is the residual buffer) and the
    residual gradient accumulated into dx in place: equal to the out-of-place
    calls, bitwise."""
    _say("residual in place", wl)
    inp = make_inputs(wl, seed=14)
    dims = _dims(wl)
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    res = [x.clone() for _ in range(wl.n_up)]
    y_ref, h = rb.fwd(dims, x, gamma, A, B, residual=res)
    ws = rb.workspace(dims, False)
    rb.lr_block_fwd_residual(dims, x, gamma, A, B, res, res, None, None, ws)   # y_i written over residual_i
    dy = [dev(t) for t in inp.dy]
    g_ref = rb.bwd(dims, x, gamma, A, B, h, dy, dx_residual=dy[0])
    dx = dy[0].clone()
    dgamma = torch.empty(wl.d, dtype=torch.float32, device="cuda")
    dA = torch.empty((wl.d, wl.g * wl.r), dtype=torch.float32, device="cuda")
    dB = [torch.empty((wl.r, wl.d), dtype=torch.float32, device="cuda") for _ in range(wl.n_up)]
    rb.lr_block_bwd_residual(dims, x, gamma, A, B, h, None, dy, dx, dx, dgamma, dA, dB, rb.workspace(dims, True))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(res, y_ref))
    assert torch.equal(dx, g_ref["dx"]) and torch.equal(dA, g_ref["dA"]) and torch.equal(dgamma, g_ref["dgamma"])


def workloads_tensor(values64, dtype):
    from workloads import Tensor
    return Tensor(values64, dtype)


def test_full_size_residual_sublayer():
    """The SwiGLU sublayer out = x + block(x) at its full shape: sampled forward
    rows, every gradient whole (dx including dy through the residual)."""
    wl = WORKLOADS["swiglu_mlp_res"]
    _say("full residual", wl)
    inp = make_inputs(wl, seed=0)
    dims = _dims(wl)
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    rstd = torch.empty(wl.T, dtype=torch.float32, device="cuda")
    y, h = rb.fwd(dims, x, gamma, A, B, rstd=rstd, residual=[x])
    dy = [dev(t) for t in inp.dy]
    g = rb.bwd(dims, x, gamma, A, B, h, dy, rstd=rstd, dx_residual=dy[0])
    torch.cuda.synchronize()
    rows = _sample_rows(wl.T)
    ri = torch.as_tensor(rows, device="cuda")
    Bv = [b.v for b in inp.B]
    ref = oracle.block_fwd(inp.x.v[rows], inp.gamma.v, inp.A.v, Bv, wl.r, wl.g, wl.act, wl.eps, wl.D,
                           residual=[inp.x.v[rows]])
    assert_close(host(y[0][ri]), ref["y"][0], wl.dtype, "y0 rows")
    del y
    rbw = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, Bv, [t.v for t in inp.dy], wl.r, wl.g, wl.act, wl.eps,
                           wl.D, dx_residual=inp.dy[0].v)
    for k in ("dx", "dgamma", "dA"):
        assert_close(host(g[k]), rbw[k], wl.dtype, k)
    assert_close(host(g["dB"][0]), rbw["dB"][0], wl.dtype, "dB0")


@pytest.mark.parametrize("wl", [
    # 384 weight-gradient tiles: 128 dB tiles run as two token halves, 256 whole
    Workload("bf16_wgrad_split_tiles", 2048, 4096, 1024, 3, "silu", "bf16"),
    # ragged: partial rank tiles (r = 960), T not a multiple of the k step
    Workload("bf16_wgrad_split_tiles_ragged", 2050, 4096, 960, 3, "identity", "bf16"),
], ids=lambda w: w.name)
def test_backward_split_tiles(wl):
    """Weight gradients that split only some (dB) tiles over two token halves:
    every gradient compared whole."""
    _say("split tiles bwd", wl)
    inp = make_inputs(wl, seed=15)
    dims, (x, gamma, A, B), y, h = _run_fwd(wl, inp)
    g = rb.bwd(dims, x, gamma, A, B, h, [dev(t) for t in inp.dy])
    torch.cuda.synchronize()
    ref = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], [t.v for t in inp.dy],
                           wl.r, wl.g, wl.act, wl.eps, wl.D)
    for k in ("dx", "dgamma", "dA"):
        assert_close(host(g[k]), ref[k], wl.dtype, k)
    for i in range(len(B)):
        assert_close(host(g["dB"][i]), ref["dB"][i], wl.dtype, f"dB{i}")


@pytest.mark.parametrize("wl", [
    # 891 up-projection tiles (3.5 rounds), ragged T, a partial last column tile
    # (d = 2112), K = 320 (five k steps)
    Workload("bf16_up_many_tiles_ragged", 8269, 2112, 320, 3, "silu", "bf16"),
    # SwiGLU's single up-projection, 1024 tiles
    Workload("bf16_up_many_tiles_swiglu", 4096, 4096, 512, 2, "swiglu", "bf16"),
], ids=lambda w: w.name)
def test_forward_up_many_tiles(wl):
    """Up-projections over several rounds of tiles with ragged edges: h and
    every y_i compared whole."""
    _say("up many tiles", wl)
    inp = make_inputs(wl, seed=16, with_dy=False)
    _, _, y, h = _run_fwd(wl, inp)
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(h), ref["h"], wl.dtype, "h")
    for i, yi in enumerate(y):
        assert_close(host(yi), ref["y"][i], wl.dtype, f"y{i}")


def test_degenerate_rows():
    """RMSNorm's degenerate rows through the whole block: all-zero rows (rstd =
    eps^-1/2, h = 0), constant rows, rows scaled by 1e3 and 1e-3 (the statistic
    spans 12 orders of magnitude), each against the oracle on the same bf16
    values; forward and backward (a ragged T over several tiles)."""
    from workloads import Tensor
    wl = Workload("bf16_degenerate", 700, 512, 128, 3, "silu", "bf16")
    _say("degenerate rows", wl)
    inp = make_inputs(wl, seed=9)
    xv = inp.x.v.copy()
    xv[0] = 0.0
    xv[5] = 0.0
    xv[299] = 1.5
    xv[300] = -0.25
    xv[301:305] *= 1e3
    xv[305:309] *= 1e-3
    xv[-1] = 0.0
    inp.x = Tensor(xv, wl.dtype)
    dims, (x, gamma, A, B), y, h = _run_fwd(wl, inp)
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(h), ref["h"], wl.dtype, "h")
    for i, yi in enumerate(y):
        assert_close(host(yi), ref["y"][i], wl.dtype, f"y{i}")
    g = rb.bwd(dims, x, gamma, A, B, h, [dev(t) for t in inp.dy])
    torch.cuda.synchronize()
    rb_ = oracle.block_bwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], [t.v for t in inp.dy],
                           wl.r, wl.g, wl.act, wl.eps, wl.D)
    for k in ("dx", "dgamma", "dA"):
        assert_close(host(g[k]), rb_[k], wl.dtype, k)
    for i in range(len(B)):
        assert_close(host(g["dB"][i]), rb_["dB"][i], wl.dtype, f"dB{i}")
    # the zero rows' outputs: h = 0 exactly, y = SiLU(0) . B = 0 exactly
    assert torch.count_nonzero(h[0]).item() == 0 and torch.count_nonzero(y[0][0]).item() == 0


def test_graph_capture_replays_match_eager():
    """The library allocates nothing and records no memsets, so its launches can
    be captured in a HIP graph: one fwd+bwd step (the benchmark's calls, with
    the allocation-free forward) captured once and replayed four times, with
    eager work and synchronisation between the replays; every replay equals the
    eager step bit for bit (same kernels, same order)."""
    wl = Workload("bf16_graph", 1100, 512, 256, 3, "silu", "bf16")
    _say("graph capture", wl)
    inp = make_inputs(wl, seed=12)
    dims = _dims(wl)
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    dy = [dev(t) for t in inp.dy]
    dt = torch.bfloat16
    y = [torch.empty(wl.T, wl.d, dtype=dt, device="cuda") for _ in range(3)]
    h = torch.empty(wl.T, wl.g * wl.r, dtype=dt, device="cuda")
    rstd = torch.empty(wl.T, dtype=torch.float32, device="cuda")
    dx = torch.empty(wl.T, wl.d, dtype=dt, device="cuda")
    dgamma = torch.empty(wl.d, dtype=torch.float32, device="cuda")
    dA = torch.empty(wl.d, wl.g * wl.r, dtype=torch.float32, device="cuda")
    dB = [torch.empty(wl.r, wl.d, dtype=torch.float32, device="cuda") for _ in range(3)]
    wsb = rb.workspace(dims, True)

    def step():
        rb.lr_block_fwd_noalloc(dims, x, gamma, A, B, y, h, rstd)
        rb.lr_block_bwd_rstd(dims, x, gamma, A, B, h, rstd, dy, dx, dgamma, dA, dB, wsb)

    outs = lambda: [t.clone() for t in [*y, h, rstd, dx, dgamma, dA, *dB]]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # the first call looks the scratch address up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = outs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for t in [*y, h, rstd, dx, dgamma, dA, *dB]:
            t.fill_(float("nan"))   # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), eager):
            assert torch.equal(a, b), f"replay {i}"
    ref = oracle.block_fwd(inp.x.v, inp.gamma.v, inp.A.v, [b.v for b in inp.B], wl.r, wl.g, wl.act, wl.eps, wl.D)
    assert_close(host(y[0]), ref["y"][0], wl.dtype, "y0 (graph)")
