"""The allocation-free forward (lr_block_fwd_noalloc) through the C ABI against
the workspace forward (lr_block_fwd_rstd): two calls in a row, the second on a
smaller input (and another path), each bitwise equal to the workspace
forward's output, which meets the oracle-parity bar of that entry point."""
import sys

import pytest
import torch

import rank_bottleneck_amd as rb
from workloads import Workload, make_inputs

from util import dev

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[no-alloc]", *a, file=sys.stderr, flush=True)


def _both(wl, seed):
    inp = make_inputs(wl, seed=seed, with_dy=False)
    dims = rb.make_dims(wl.T, wl.d, wl.r, wl.g, wl.act, wl.dtype, wl.eps)
    x, gamma, A = dev(inp.x), dev(inp.gamma), dev(inp.A)
    B = [dev(b) for b in inp.B]
    dt = rb.TORCH_DTYPE[dims.dtype]
    nu = rb.n_up(dims)

    def outs():
        y = [torch.full((wl.T, wl.d), float("nan"), dtype=dt, device="cuda") for _ in range(nu)]
        h = torch.full((wl.T, wl.g * wl.r), float("nan"), dtype=dt, device="cuda")
        rs = torch.full((wl.T,), float("nan"), dtype=torch.float32, device="cuda")
        return y, h, rs

    y0, h0, r0 = outs()
    rb.lr_block_fwd_rstd(dims, x, gamma, A, B, y0, h0, r0, rb.workspace(dims, False))
    y1, h1, r1 = outs()
    rb.lr_block_fwd_noalloc(dims, x, gamma, A, B, y1, h1, r1)
    torch.cuda.synchronize()
    assert torch.equal(h0, h1), "h"
    assert torch.equal(r0, r1), "rstd"
    for i in range(nu):
        assert torch.equal(y0[i], y1[i]), f"y{i}"


def test_noalloc_forward_two_calls_second_smaller():
    # first: the two-kernel GEMM path, z through the scratch (ragged T)
    big = Workload("noalloc_big", 4099, 1024, 512, 3, "silu", "bf16")
    _say("first call", big)
    _both(big, 21)
    # second, smaller: the one-kernel small-rank path (A'^T and B in fragment
    # order in the scratch), then the split-K small-rank path (fp32 partials)
    small = Workload("noalloc_small", 777, 512, 64, 2, "swiglu", "bf16")
    _say("second call", small)
    _both(small, 22)
    split = Workload("noalloc_split", 300, 384, 192, 1, "silu", "bf16")
    _say("third call", split)
    _both(split, 23)


def test_noalloc_rejects_oversize_without_launching():
    dims = rb.make_dims(65536, 4096, 1024, 3, "silu", "bf16")
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rb.LrError) as e:
        rb.lr_block_fwd_noalloc(dims, x, x, x, [x, x, x], [x, x, x], None, None)
    assert e.value.status == rb.LR_EWORKSPACE
