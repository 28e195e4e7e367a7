"""The C ABI without a GPU: the library loads, exports every symbol that
include/lr_block.h declares, sizes workspaces, and rejects bad arguments on the
host (returning a status, launching nothing)."""
import ctypes
import os
import re

import pytest

import rank_bottleneck_amd as rb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lr_block.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rb.LIB_PATH), reason="liblrblock.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(rb.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = rb.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert rb.lr_status_str(rb.LR_OK) == "LR_OK"
    assert rb.lr_status_str(rb.LR_EWORKSPACE) == "LR_EWORKSPACE"
    assert rb.lr_status_str(99) == "LR_UNKNOWN"


def test_workspace_sizes():
    d = rb.make_dims(16384, 4096, 1024, 3, "silu", "bf16")
    f, b = rb.lr_block_workspace_size(d, False), rb.lr_block_workspace_size(d, True)
    # forward: gamma-folded A plus sigma(h); backward: rstd, dh', sigma(h), row partials
    assert f >= 4096 * 3072 * 2 + 16384 * 3072 * 2
    assert b >= 16384 * 4 + 2 * 16384 * 3072 * 2
    assert rb.lr_block_workspace_size(rb.make_dims(16, 100, 64, 1), False) == 0   # d % 64 != 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails its host checks


def _call_fwd(dims, x=FAKE, gamma=FAKE, A=FAKE, nB=None, h=None, rstd=None, ws=FAKE, ws_bytes=1 << 40,
              form="plain"):
    """lr_block_fwd (the scope table's signature, no rstd) or, with form="rstd",
    lr_block_fwd_rstd; both must give the same status."""
    lib = rb.load()
    n = rb.n_up(dims) if nB is None else nB
    B = (ctypes.c_void_p * max(n, 1))(*([FAKE] * n))
    y = (ctypes.c_void_p * max(n, 1))(*([FAKE] * n))
    if form == "plain":
        assert rstd is None
        return lib.lr_block_fwd(ctypes.byref(dims), x, gamma, A, B, y, h, ws, ws_bytes, None)
    return lib.lr_block_fwd_rstd(ctypes.byref(dims), x, gamma, A, B, y, h, rstd, ws, ws_bytes, None)


FORMS = pytest.mark.parametrize("form", ["plain", "rstd"])


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), rb.LR_EINVAL),
    (dict(d=100), rb.LR_EUNSUPPORTED),
    (dict(r=96), rb.LR_EUNSUPPORTED),
    (dict(g=9), rb.LR_EUNSUPPORTED),
    (dict(g=3, act="swiglu"), rb.LR_EUNSUPPORTED),
    (dict(eps=float("nan")), rb.LR_EINVAL),
    (dict(eps=-1.0), rb.LR_EINVAL),
])
@FORMS
def test_bad_dims_rejected(kw, status, form):
    args = dict(T=64, d=128, r=64, g=1, act="silu", dtype="bf16", eps=1e-6)
    args.update(kw)
    dims = rb.make_dims(**args)
    assert _call_fwd(dims, form=form) == status


@FORMS
def test_bad_enums_rejected(form):
    dims = rb.make_dims(64, 128, 64, 1)
    dims.dtype = 7
    assert _call_fwd(dims, form=form) == rb.LR_EINVAL
    dims = rb.make_dims(64, 128, 64, 1)
    dims.act = 5
    assert _call_fwd(dims, form=form) == rb.LR_EINVAL
    lib = rb.load()
    assert lib.lr_block_fwd(None, FAKE, FAKE, FAKE, None, None, None, FAKE, 1, None) == rb.LR_EINVAL
    assert lib.lr_block_fwd_rstd(None, FAKE, FAKE, FAKE, None, None, None, None, FAKE, 1, None) == rb.LR_EINVAL


@FORMS
def test_bad_pointers_rejected(form):
    dims = rb.make_dims(64, 128, 64, 2, "identity")
    assert _call_fwd(dims, x=None, form=form) == rb.LR_EINVAL
    assert _call_fwd(dims, A=FAKE + 2, form=form) == rb.LR_EINVAL           # misaligned
    assert _call_fwd(dims, h=FAKE + 8, form=form) == rb.LR_EINVAL
    assert _call_fwd(dims, nB=1, form=form) == rb.LR_EINVAL                 # second B pointer null
    if form == "rstd":
        assert _call_fwd(dims, rstd=FAKE + 4, form=form) == rb.LR_EINVAL


def test_workspace_checked():
    dims = rb.make_dims(64, 128, 64, 1)
    need = rb.lr_block_workspace_size(dims, False)
    for form in ("plain", "rstd"):
        assert _call_fwd(dims, ws=None, form=form) == rb.LR_EWORKSPACE
        assert _call_fwd(dims, ws_bytes=need - 1, form=form) == rb.LR_EWORKSPACE
    lib = rb.load()
    arr = (ctypes.c_void_p * 1)(FAKE)
    need_b = rb.lr_block_workspace_size(dims, True)
    # lr_block_bwd: the scope table's signature (no rstd argument)
    assert lib.lr_block_bwd(ctypes.byref(dims), FAKE, FAKE, FAKE, arr, FAKE, arr, FAKE, FAKE, FAKE, arr,
                            FAKE, need_b - 1, None) == rb.LR_EWORKSPACE
    assert lib.lr_block_bwd(ctypes.byref(dims), FAKE, FAKE, FAKE, arr, None, arr, FAKE, FAKE, FAKE, arr,
                            FAKE, 1 << 40, None) == rb.LR_EINVAL   # h_saved missing
    assert lib.lr_block_bwd_rstd(ctypes.byref(dims), FAKE, FAKE, FAKE, arr, FAKE, None, arr, FAKE, FAKE, FAKE, arr,
                                 FAKE, need_b - 1, None) == rb.LR_EWORKSPACE
    assert lib.lr_block_bwd_rstd(ctypes.byref(dims), FAKE, FAKE, FAKE, arr, FAKE, FAKE + 4, arr, FAKE, FAKE, FAKE,
                                 arr, FAKE, 1 << 40, None) == rb.LR_EINVAL   # misaligned rstd_saved
    assert lib.lr_down_partial(ctypes.byref(dims), FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None) == rb.LR_EINVAL
    assert lib.lr_up_finish(ctypes.byref(dims), FAKE, FAKE, arr, arr, None, None, 0, None) == rb.LR_EWORKSPACE


def test_trace_arguments():
    assert rb.load().lr_trace_begin(None, 0) == rb.LR_EINVAL
    assert rb.load().lr_trace_begin(None, (1 << 16) + 1) == rb.LR_EINVAL   # capped, nothing allocated
    assert rb.lr_trace_count() == 0


def test_rmsnorm_arguments():
    lib = rb.load()
    dims = rb.make_dims(8, 12, 64, 1)
    assert lib.rmsnorm_online(ctypes.byref(dims), FAKE, FAKE, None, None, None, None) == rb.LR_EUNSUPPORTED
    dims = rb.make_dims(8, 16, 64, 1)
    assert lib.rmsnorm_online(ctypes.byref(dims), None, FAKE, None, None, None, None) == rb.LR_EINVAL
    assert lib.rmsnorm_online(ctypes.byref(dims), FAKE, None, FAKE, None, None, None) == rb.LR_EINVAL


def test_noalloc_rejects_on_the_host():
    """lr_block_fwd_noalloc's checks that run before any HIP call: bad dims and
    pointers, and dims whose workspace exceeds the static scratch."""
    lib = rb.load()
    arr = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    big = rb.make_dims(65536, 4096, 1024, 3, "silu", "bf16")          # 25 MiB + 384 MiB
    assert rb.lr_block_workspace_size(big, False) > rb.NOALLOC_SCRATCH_BYTES
    assert lib.lr_block_fwd_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, arr, arr, None, None, None) \
        == rb.LR_EWORKSPACE
    c4 = rb.make_dims(16384, 4096, 1024, 3, "silu", "bf16")           # the largest forward here fits
    assert rb.lr_block_workspace_size(c4, False) <= rb.NOALLOC_SCRATCH_BYTES
    bad = rb.make_dims(64, 100, 64, 1)
    assert lib.lr_block_fwd_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, arr, arr, None, None, None) \
        == rb.LR_EUNSUPPORTED
    ok = rb.make_dims(64, 128, 64, 1)
    assert lib.lr_block_fwd_noalloc(ctypes.byref(ok), None, FAKE, FAKE, arr, arr, None, None, None) == rb.LR_EINVAL
    assert lib.lr_block_fwd_noalloc(ctypes.byref(ok), FAKE, FAKE, FAKE, arr, arr, None, FAKE + 4, None) \
        == rb.LR_EINVAL


def declared_signatures():
    """{name: number of parameters} of every function the header declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(([^)]*)\)\s*;", src, flags=re.M):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argtypes_match_the_header():
    """Every entry point's ctypes argument list has as many entries as the C
    declaration has parameters (a short list would pass later arguments, the
    stream among them, with ctypes' default int conversion)."""
    lib = rb.load()
    sig = declared_signatures()
    assert sorted(sig) == sorted(rb.ENTRY_POINTS)
    for name, n in sig.items():
        assert len(getattr(lib, name).argtypes) == n, name


def test_mlp_host_checks():
    lib = rb.load()
    m = rb.make_mlp_dims(16384, 4096, 11008, 1024)
    f, b = rb.lr_mlp_workspace_size(m, False), rb.lr_mlp_workspace_size(m, True)
    # forward: folded A_in, h_in, h_out, gate and s; backward: gate, up, s and more
    assert f >= 4096 * 2048 * 2 + 16384 * 3072 * 2 + 2 * 16384 * 11008 * 2
    assert b >= 3 * 16384 * 11008 * 2
    assert rb.lr_mlp_workspace_size(rb.make_mlp_dims(64, 128, 100, 64), False) == 0    # f % 64
    ok = rb.make_mlp_dims(64, 128, 192, 64)
    need = rb.lr_mlp_workspace_size(ok, False)
    p = [FAKE] * 7
    assert lib.lr_mlp_fwd(ctypes.byref(ok), *p, None, FAKE, None, None, None, FAKE, need - 1, None) \
        == rb.LR_EWORKSPACE
    assert lib.lr_mlp_fwd(ctypes.byref(ok), *p, None, None, None, None, None, FAKE, need, None) \
        == rb.LR_EINVAL                                                                  # out missing
    assert lib.lr_mlp_fwd(ctypes.byref(ok), *p, FAKE + 2, FAKE, None, None, None, FAKE, need, None) \
        == rb.LR_EINVAL                                                                  # misaligned residual
    bad = rb.make_mlp_dims(64, 128, 192, 96)
    assert lib.lr_mlp_fwd(ctypes.byref(bad), *p, None, FAKE, None, None, None, FAKE, 1 << 40, None) \
        == rb.LR_EUNSUPPORTED
    need_b = rb.lr_mlp_workspace_size(ok, True)
    g = [FAKE] * 7
    assert lib.lr_mlp_bwd(ctypes.byref(ok), *p, FAKE, FAKE, None, FAKE, None, *g, FAKE, need_b - 1, None) \
        == rb.LR_EWORKSPACE
    assert lib.lr_mlp_bwd(ctypes.byref(ok), *p, None, FAKE, None, FAKE, None, *g, FAKE, need_b, None) \
        == rb.LR_EINVAL                                                                  # h_in_saved missing
