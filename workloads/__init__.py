"""Seeded synthetic workloads for the low-rank bottleneck block.

This module only *draws* inputs; it holds none of the block's arithmetic.  Both
the CPU oracle and the HIP path are fed from it, so that the two see identical
bits.  The shapes are those of one transformer block's low-rank bottleneck in
the LLaMA-2 family that the BOOST pages evaluate on ("BOOST: BOttleneck-
Optimized Scalable Training Framework for Low-Rank Large Language Models",
technical summary §4 "Experimental results"); the pages give no sizes, so the
widths here are LLaMA-2-style (d = 2048 / 4096, ffn = 11008) with ranks
r = d/4 .. d/16.

Draw recipe (fixed order, one PCG64 stream per (config, seed)):
    x    ~ N(0, 1)            [T, d]
    gamma = 1 + N(0, 0.1)     [d]        (0.1 is a variance)
    A    ~ N(0, 1/d_w)        [d, g*r]   (d_w = d, or the unsharded width)
    B_i  ~ N(0, 1/r)          [r, d]     for i < n_up
    dy_i ~ N(0, 1)            [T, d]     for i < n_up
Every value is then rounded to the storage dtype: fp64 -> fp32 (RNE) -> bf16
(RNE) for bf16 workloads; fp64 -> fp32 for fp32 workloads.  The float64 arrays
handed to the oracle hold exactly those rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

ACTS = ("identity", "silu", "swiglu")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    r: int
    g: int
    act: str
    dtype: str            # "f32" or "bf16"
    eps: float = 1e-6
    d_norm: int = 0       # 0 -> d ; the unsharded width for a tensor-parallel shard
    d_weight: int = 0     # width used for A's init variance; 0 -> d
    seam: bool = False    # run through the shard seam (partial + finish) instead of the fused block
    fwd_only: bool = False  # benchmarked as a forward pass
    hbm_metric: bool = False  # reported as forward HBM GB/s (memory-bound sweep) instead of TFLOP/s
    residual: bool = False  # the sublayer out = x + block(x): residual_0 = x, and dx gains dy_0
    note: str = ""

    @property
    def n_up(self) -> int:
        return 1 if self.act == "swiglu" else self.g

    @property
    def D(self) -> int:
        return self.d_norm if self.d_norm else self.d

    def fwd_flops(self) -> float:
        return 2.0 * self.T * self.d * self.g * self.r + 2.0 * self.T * self.r * self.d * self.n_up

    def bwd_flops(self) -> float:
        return 4.0 * self.T * self.r * self.d * self.n_up + 4.0 * self.T * self.d * self.g * self.r

    def fwd_bytes(self) -> float:
        """Bytes a forward pass must move at least: x, gamma, A, the B_i, the y_i
        and the saved rank-r pre-activation."""
        e = 2 if self.dtype == "bf16" else 4
        gr = self.g * self.r
        return float(e * (self.T * self.d + self.d + self.d * gr + self.n_up * self.r * self.d
                          + self.n_up * self.T * self.d + self.T * gr))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32_silu": Workload("tiny_f32_silu", T=128, d=256, r=64, g=1, act="silu", dtype="f32",
                              note="b=2, s=64"),
    "qkv_identity": Workload("qkv_identity", T=16384, d=2048, r=512, g=3, act="identity", dtype="bf16",
                             note="b=8, s=2048; Q/K/V down-projections fused into one [2048,1536] GEMM"),
    "swiglu_mlp": Workload("swiglu_mlp", T=16384, d=4096, r=1024, g=2, act="swiglu", dtype="bf16",
                           note="gate/up grouped (g=2), SiLU(gate)*up at rank r, one r->d up-projection; "
                                "replaces a d=4096, ffn=11008 MLP"),
    "btp_shard": Workload("btp_shard", T=8192, d=2048, r=2048, g=1, act="silu", dtype="bf16",
                          d_norm=8192, d_weight=8192, seam=True,
                          note="one of four shards of a d=8192, r=2048 block: x[:, 2048-slice], "
                               "A row-slice, fp32 partial, B column-slice"),
    "qkv_silu_ckpt": Workload("qkv_silu_ckpt", T=16384, d=4096, r=1024, g=3, act="silu", dtype="bf16",
                              note="backward from the saved [T, 3r] pre-activation"),
}
# the SwiGLU bottleneck as a pre-norm sublayer: out = x + block(x), the residual
# add fused into the up-projection's epilogue and dy added into dx
WORKLOADS["swiglu_mlp_res"] = Workload("swiglu_mlp_res", T=16384, d=4096, r=1024, g=2, act="swiglu", dtype="bf16",
                                       residual=True,
                                       note="swiglu_mlp as the sublayer out = x + block(x) (residual fused)")
# memory-bound small-rank sweep (forward)
for _r in (64, 128, 256):
    WORKLOADS[f"small_r{_r}"] = Workload(f"small_r{_r}", T=16384, d=4096, r=_r, g=1, act="silu",
                                         dtype="bf16", fwd_only=True, hbm_metric=True)
# the same sweep for a SwiGLU bottleneck: gate and up grouped (g = 2) at rank r
for _r in (64, 128):
    WORKLOADS[f"small_swiglu_r{_r}"] = Workload(f"small_swiglu_r{_r}", T=16384, d=4096, r=_r, g=2, act="swiglu",
                                                dtype="bf16", fwd_only=True, hbm_metric=True)
# contrast to btp_shard: the same d=8192, r=2048 block under vanilla low-rank TP=4
WORKLOADS["vanilla_tp_shard"] = Workload(
    "vanilla_tp_shard", T=8192, d=8192, r=512, g=1, act="silu", dtype="bf16", fwd_only=True,
    note="one of four vanilla tensor-parallel shards of the d=8192, r=2048 block: A column slice [8192, 512], "
         "B row slice [512, 8192]; y is a [T, d] partial (the all-reduce payload). Same FLOPs as btp_shard, "
         "but the up-projection's K is r/4 = 512")


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round to bf16 (fp64 -> fp32 RNE -> bf16 RNE); returns uint16 bit patterns."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


class Tensor:
    """One input array: its exact float64 values and its storage representation."""

    def __init__(self, values64: np.ndarray, dtype: str):
        self.dtype = dtype
        if dtype == "bf16":
            self.store = bf16_bits(values64)            # uint16
            self.v = bf16_to_f64(self.store)
        elif dtype == "f32":
            self.store = np.ascontiguousarray(values64, dtype=np.float32)
            self.v = self.store.astype(np.float64)
        else:
            raise ValueError(dtype)

    @property
    def shape(self):
        return self.v.shape


@dataclasses.dataclass
class Inputs:
    wl: Workload
    seed: int
    x: Tensor
    gamma: Tensor
    A: Tensor
    B: List[Tensor]
    dy: Optional[List[Tensor]]


def make_inputs(wl: Workload, seed: int = 0, with_dy: bool = True, rows: Optional[int] = None) -> Inputs:
    """Draw one workload's inputs.  ``rows`` (<= T) keeps only the first rows of
    x and dy *after* drawing the full arrays, so a row subset has the same
    values as the full draw."""
    rng = np.random.default_rng(seed)
    T, d, r, g = wl.T, wl.d, wl.r, wl.g
    dw = wl.d_weight if wl.d_weight else d
    keep = T if rows is None else min(rows, T)
    x = rng.standard_normal((T, d))[:keep]
    gamma = 1.0 + rng.standard_normal(d) * math.sqrt(0.1)
    A = rng.standard_normal((d, g * r)) / math.sqrt(dw)
    B = [rng.standard_normal((r, d)) / math.sqrt(r) for _ in range(wl.n_up)]
    dy = None
    if with_dy:
        dy = [rng.standard_normal((T, d))[:keep] for _ in range(wl.n_up)]
    dt = wl.dtype
    return Inputs(wl, seed, Tensor(x, dt), Tensor(gamma, dt), Tensor(A, dt),
                  [Tensor(b, dt) for b in B], None if dy is None else [Tensor(t, dt) for t in dy])


# ----------------------------------------------------------------------------- per-projection MLP
@dataclasses.dataclass(frozen=True)
class MlpWorkload:
    """The per-projection low-rank SwiGLU MLP: model width d, MLP width f, every
    factorised linear of rank r."""
    name: str
    T: int
    d: int
    f: int
    r: int
    dtype: str
    eps: float = 1e-6
    residual: bool = False   # out = x + mlp(x): residual = x, and dx gains dout
    note: str = ""

    def fwd_flops(self) -> float:
        """GEMMs of a forward: x . A_in, the two up factors to f, s . A_o, h_out . B_o."""
        return 2.0 * self.T * self.r * (3 * self.d + 3 * self.f)

    def bwd_flops(self) -> float:
        """GEMMs of a backward, without the recomputation of gate and up (two
        more up factors, 4 T r f)."""
        return 2.0 * self.T * self.r * (6 * self.d + 6 * self.f)

    def recompute_flops(self) -> float:
        return 4.0 * self.T * self.r * self.f

    def replace(self, **kw) -> "MlpWorkload":
        return dataclasses.replace(self, **kw)


MLP_WORKLOADS: Dict[str, MlpWorkload] = {
    "lowrank_mlp": MlpWorkload("lowrank_mlp", T=16384, d=4096, f=11008, r=1024, dtype="bf16", residual=True,
                               note="LLaMA-2-7B-width MLP sublayer out = x + mlp(x), each of gate, up and down "
                                    "a rank-1024 factor pair, SwiGLU at width 11008"),
}


@dataclasses.dataclass
class MlpInputs:
    wl: MlpWorkload
    seed: int
    x: Tensor
    gamma: Tensor
    A_in: Tensor
    B_g: Tensor
    B_u: Tensor
    A_o: Tensor
    B_o: Tensor
    dout: Optional[Tensor]


def make_mlp_inputs(wl: MlpWorkload, seed: int = 0, with_dout: bool = True, rows: Optional[int] = None) -> MlpInputs:
    """Draw one MLP workload's inputs (fixed order, one PCG64 stream per seed):
        x     ~ N(0, 1)          [T, d]
        gamma = 1 + N(0, 0.1)    [d]
        A_in  ~ N(0, 1/d)        [d, 2r]   ([A_g | A_u])
        B_g   ~ N(0, 1/r)        [r, f]
        B_u   ~ N(0, 1/r)        [r, f]
        A_o   ~ N(0, 1/f)        [f, r]
        B_o   ~ N(0, 1/r)        [r, d]
        dout  ~ N(0, 1)          [T, d]
    rounded to the storage dtype as for the block.  ``rows`` keeps the first
    rows of x and dout after drawing the full arrays."""
    rng = np.random.default_rng(seed)
    T, d, f, r = wl.T, wl.d, wl.f, wl.r
    keep = T if rows is None else min(rows, T)
    x = rng.standard_normal((T, d))[:keep]
    gamma = 1.0 + rng.standard_normal(d) * math.sqrt(0.1)
    A_in = rng.standard_normal((d, 2 * r)) / math.sqrt(d)
    B_g = rng.standard_normal((r, f)) / math.sqrt(r)
    B_u = rng.standard_normal((r, f)) / math.sqrt(r)
    A_o = rng.standard_normal((f, r)) / math.sqrt(f)
    B_o = rng.standard_normal((r, d)) / math.sqrt(r)
    dout = rng.standard_normal((T, d))[:keep] if with_dout else None
    dt = wl.dtype
    return MlpInputs(wl, seed, Tensor(x, dt), Tensor(gamma, dt), Tensor(A_in, dt), Tensor(B_g, dt), Tensor(B_u, dt),
                     Tensor(A_o, dt), Tensor(B_o, dt), None if dout is None else Tensor(dout, dt))
