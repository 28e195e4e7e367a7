"""bench.py's host-side logic without a GPU: the per-kernel algorithmic work
adds up to the step's, the one-GPU guard, and the checkpoint figure."""
import os
import subprocess
import sys

import pytest

import bench
from workloads import MLP_WORKLOADS, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name", ["qkv_identity", "swiglu_mlp", "qkv_silu_ckpt", "swiglu_mlp_res"])
def test_block_kernel_flops_add_up(name):
    """down + up = the forward's GEMM flops; dz + wgrad + dx = the backward's."""
    wl = WORKLOADS[name]
    f = lambda k: bench.kernel_work(wl, k)[0]
    assert f("down") + f("up") == pytest.approx(wl.fwd_flops(), rel=1e-12)
    assert f("dz") + f("wgrad") + f("dx") == pytest.approx(wl.bwd_flops(), rel=1e-12)


def test_mlp_kernel_flops_add_up():
    """The MLP's kernels, summed over their launches in a step, execute the
    forward, the backward and the recomputation of gate and up."""
    wl = MLP_WORKLOADS["lowrank_mlp"]
    total = sum(bench.mlp_kernel_work(wl, k)[0] for k in ("up", "down", "dz", "wgrad", "dx"))
    assert total == pytest.approx(wl.fwd_flops() + wl.bwd_flops() + wl.recompute_flops(), rel=1e-12)


def test_fused_forward_bytes_are_each_tensor_once():
    wl = WORKLOADS["small_r64"]
    assert bench.kernel_work(wl, "fused")[1] == wl.fwd_bytes() - 2 * wl.d   # gamma is folded, not read


def test_checkpoint_figure():
    c = bench.checkpoint_bytes(WORKLOADS["qkv_silu_ckpt"])
    assert c["kept_bytes"] == 2 * 16384 * 3072 + 4 * 16384
    assert c["ratio"] > 3


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr
