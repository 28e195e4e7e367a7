"""The seeded input generator: determinism, bf16 round-to-nearest-even, the
draw recipe's moments, and that a row subset equals the full draw's rows."""
import numpy as np
import torch

from workloads import WORKLOADS, bf16_bits, bf16_to_f64, make_inputs


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40]])
    ours = bf16_bits(v)
    ref = torch.tensor(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert bf16_to_f64(bf16_bits(np.array([1.0 + 2.0 ** -8])))[0] == 1.0
    assert bf16_to_f64(bf16_bits(np.array([1.0 + 3 * 2.0 ** -8])))[0] == 1.0 + 2.0 ** -6


def test_deterministic_and_row_subset():
    wl = WORKLOADS["tiny_f32_silu"]
    a = make_inputs(wl, 0)
    b = make_inputs(wl, 0)
    c = make_inputs(wl, 0, rows=17)
    assert np.array_equal(a.x.v, b.x.v) and np.array_equal(a.A.v, b.A.v)
    assert np.array_equal(a.x.v[:17], c.x.v) and np.array_equal(a.dy[0].v[:17], c.dy[0].v)
    assert np.array_equal(a.B[0].v, c.B[0].v)
    assert not np.array_equal(make_inputs(wl, 1).x.v, a.x.v)


def test_recipe_moments():
    wl = WORKLOADS["qkv_identity"].replace(T=512)
    inp = make_inputs(wl, 0)
    d, r = wl.d, wl.r
    assert abs(inp.x.v.std() - 1.0) < 0.01
    assert abs(inp.A.v.std() * np.sqrt(d) - 1.0) < 0.01
    assert abs(inp.B[0].v.std() * np.sqrt(r) - 1.0) < 0.01
    assert abs((inp.gamma.v - 1.0).std() - np.sqrt(0.1)) < 0.03
    assert inp.x.store.dtype == np.uint16 and len(inp.B) == 3 and len(inp.dy) == 3
    assert WORKLOADS["swiglu_mlp"].n_up == 1


def test_mlp_inputs_deterministic_and_recipe():
    from workloads import MLP_WORKLOADS, make_mlp_inputs
    wl = MLP_WORKLOADS["lowrank_mlp"].replace(T=256, d=512, f=1024, r=128)
    a, b, c = make_mlp_inputs(wl, 0), make_mlp_inputs(wl, 0), make_mlp_inputs(wl, 0, rows=33)
    for k in ("x", "gamma", "A_in", "B_g", "B_u", "A_o", "B_o", "dout"):
        assert np.array_equal(getattr(a, k).v, getattr(b, k).v), k
    assert np.array_equal(a.x.v[:33], c.x.v) and np.array_equal(a.dout.v[:33], c.dout.v)
    assert np.array_equal(a.A_o.v, c.A_o.v)
    assert a.A_in.shape == (512, 256) and a.B_g.shape == (128, 1024) and a.A_o.shape == (1024, 128)
    assert a.B_o.shape == (128, 512) and a.x.store.dtype == np.uint16
    assert abs(a.A_in.v.std() * np.sqrt(512) - 1.0) < 0.02
    assert abs(a.A_o.v.std() * np.sqrt(1024) - 1.0) < 0.02
    assert abs(a.B_g.v.std() * np.sqrt(128) - 1.0) < 0.02
    assert not np.array_equal(make_mlp_inputs(wl, 1).x.v, a.x.v)
