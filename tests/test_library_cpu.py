"""The C-ABI library loads on a CPU-only host, exports every symbol the
header declares, and rejects invalid arguments before touching a device."""

import ctypes
import math
import os
import re

import pytest

import token_early_exit_amd as tee

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(river_[a-z_0-9]+)\s*\(", src))
    return names


def test_exports_every_declared_symbol():
    lib = tee.load()
    declared = _declared_functions()
    assert {"river_route", "river_compact", "river_kv_fill", "river_ridge_fit"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(tee.EXPORTS) == declared


def test_version_and_error_string():
    assert tee.version().startswith("river")
    assert tee.load().river_last_error() is not None


def test_kernel_timing_hook_rejects_unknown_kinds():
    """The timing switch only sets a flag (no device call); reading an
    unknown launch kind is an argument error before any device call."""
    tee.river_debug_time_kernels(False)
    for kind in (-1, 2, 99):
        with pytest.raises(RuntimeError, match="ERR_ARG"):
            tee.river_debug_kernel_times(kind)


def test_workspace_sizes():
    ws = tee.river_workspace_size
    assert ws(tee.OP_ROUTE, 4096, 768) == 0
    assert ws(tee.OP_KV_FILL, 4096, 768, 0, 0, 0) == 0           # identity: none
    assert ws(tee.OP_KV_FILL, 4096, 768, 0, 0, 8) >= 8 * 4096 * 768 * 2
    assert ws(tee.OP_COMPACT, 100000) >= 4 * 25
    assert ws(tee.OP_RIDGE_FIT, 2048, 768, 768, 8, tee.RIVER_BF16) > 0
    # folding: the dequantised weights (2 n_out x d) and the transposed map (d x d) per layer
    assert ws(tee.OP_KV_FOLD, 0, 4096, 1024, 0, 3) == 3 * (2 * 1024 * 4096 * 2 + 4096 * 4096 * 2)
    assert ws(tee.OP_KV_FOLD, 0, 4096, 1024, 0, 0) == 0
    # split reductions: up to 64 rows always, 65 to 256 rows when the
    # projection has few tiles (at most 128 of 64 rows x 256 outputs)
    nh = 8 * 64
    base = ws(tee.OP_KV_FILL, 200, 2048, 0, 0, 2)
    assert ws(tee.OP_KV_FILL, 200, 2048, nh, 0, 2) >= base + 2 * 200 * 2 * nh * 4 * 2
    assert ws(tee.OP_KV_FILL, 256, 4096, 1024, 0, 21) == ws(tee.OP_KV_FILL, 256, 4096, 0, 0, 21)
    assert ws(tee.OP_KV_FILL, 300, 2048, nh, 0, 1) == ws(tee.OP_KV_FILL, 300, 2048, 0, 0, 1)
    # the decode step holds the split of its smallest fill (one block)
    assert ws(tee.OP_DECODE_STEP, 256, 4096, 1024, 0, 32) > ws(tee.OP_DECODE_STEP, 256, 4096, 0, 0, 32)


def test_bench_refuses_more_than_one_gpu():
    import subprocess, sys, json, os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    assert "--gpus must be 1" in json.loads(line)["error"]


def _route(**kw):
    lib = tee.load()
    a = dict(n=4, d=64, dt=tee.RIVER_F32, hp=16, ldp=64, hc=16, ldc=64, gamma=None, eps=1e-6,
             wd=None, wu=None, b=0, tau=0.5, theta=0.5, rule=0, cos=None, prob=None, mask=16,
             all=None, s=None)
    a.update(kw)
    return lib.river_route(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), 2),
    (dict(n=-1), 1),
    (dict(d=12), 1),
    (dict(tau=math.nan), 1),
    (dict(rule=5), 1),
    (dict(eps=-1.0), 1),
    (dict(wd=16, wu=16, b=0), 1),
    (dict(wd=16, wu=None, b=32), 1),
    (dict(hp=8), 3),
    (dict(ldp=60), 1 + 2),       # ld below d -> alignment/ld error
    (dict(mask=None), 1),
])
def test_route_argument_errors(kw, status):
    assert _route(**kw) == status
    assert len(tee.load().river_last_error()) > 0


def test_kv_fill_and_ridge_argument_errors():
    lib = tee.load()
    w = tee.RiverW4(16, 16, 16, tee.RIVER_BF16, 64)
    bad = tee.RiverW4(16, 16, 16, tee.RIVER_BF16, 48)
    args = lambda **k: dict(dict(m=8, mdev=None, d=128, dt=tee.RIVER_BF16, h=16, ld=128, nrows=8,
                                 ri=None, slot=16, nl=2, maps=None, wk=ctypes.byref(w),
                                 wv=ctypes.byref(w), hk=2, hd=64, kc=16, vc=16, ns=8, ws=None,
                                 wsn=0, s=None), **k).values()
    assert lib.river_kv_fill(*args(m=0)) == 0                     # empty call
    assert lib.river_kv_fill(*args(wk=ctypes.byref(bad))) == 1     # group does not divide d
    assert lib.river_kv_fill(*args(maps=16)) == 5                  # maps need a workspace
    assert lib.river_kv_fill(*args(m=9)) == 1                      # more rows than h has
    assert lib.river_kv_fill(*args(kc=None)) == 1
    assert lib.river_kv_fill(*args(nl=70000)) == 4                 # layers past the grid limit
    r = lib.river_ridge_fit(64, 64, 64, 1, 16, tee.RIVER_BF16, 16, tee.RIVER_F32, 0.1, 16,
                            tee.RIVER_F32, 16, 1 << 30, None)
    assert r == 2                                                  # X, Y dtypes differ
    r = lib.river_ridge_fit(64, 64, 64, 1, 16, tee.RIVER_BF16, 16, tee.RIVER_BF16, -1.0, 16,
                            tee.RIVER_F32, 16, 1 << 30, None)
    assert r == 1                                                  # negative lambda
    r = lib.river_ridge_fit(64, 64, 64, 1, 16, tee.RIVER_BF16, 16, tee.RIVER_BF16, 0.1, 16,
                            tee.RIVER_F32, 16, 10, None)
    assert r == 5                                                  # workspace too small
    assert lib.river_debug_set_compact_path(9) == 1
    assert lib.river_debug_set_gemm_path(4) == 1
    assert lib.river_debug_set_decode_path(2) == 1


def test_kv_fold_and_folded_fill_argument_errors():
    lib = tee.load()
    w = tee.RiverW4(16, 16, 16, tee.RIVER_BF16, 64)
    bad = tee.RiverW4(16, 16, 16, tee.RIVER_BF16, 48)
    fold = lambda **k: lib.river_kv_fold(*dict(dict(d=256, nl=2, maps=None, wk=ctypes.byref(w),
                                                    wv=ctypes.byref(w), hk=2, hd=64, F=16, ws=None,
                                                    wsn=0, s=None), **k).values())
    assert fold(nl=0) == 0                                         # empty call
    assert fold(wk=None) == 1
    assert fold(wk=ctypes.byref(bad)) == 1                         # group does not divide d
    assert fold(d=128) == 4                                        # d % 256
    assert fold(hd=48) == 4                                        # n_out % 64
    assert fold(maps=16) == 5                                      # maps need a workspace
    assert fold(maps=16, ws=16, wsn=tee.river_workspace_size(tee.OP_KV_FOLD, 0, 256, 128, 0, 1) - 1) == 5
    assert fold(F=8) == 3
    fill = lambda **k: lib.river_kv_fill_folded(*dict(dict(m=8, mdev=None, d=256, h=16, ld=256, nrows=8,
                                                           ri=None, slot=16, nl=2, F=16, hk=2, hd=64,
                                                           kc=16, vc=16, ns=8, s=None), **k).values())
    assert fill(m=0) == 0                                          # empty call
    assert fill(d=128, ld=128) == 4                                # d % 256
    assert fill(F=None) == 1
    assert fill(m=9) == 1                                          # more rows than h has
    assert fill(ld=252) == 3                                       # ld below d
    assert fill(kc=8) == 3
    assert fill(nl=70000) == 4                                     # layers past the grid limit
    assert fill(nrows=1 << 20, m=8, ld=1024, d=1024) == 4          # h spans 2^31 bytes
    assert len(lib.river_last_error()) > 0


def _exit_projection(**kw):
    lib = tee.load()
    a = dict(m=8, mdev=None, d=64, dt=tee.RIVER_BF16, h=16, ldh=64, nrows=8, ri=None, rid=None,
             gamma=None, eps=1e-6, out=16, ldo=64, nout=8, s=None)
    a.update(kw)
    return lib.river_exit_projection(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(m=0), 0),               # empty call, nothing enqueued
    (dict(m=0, d=12), 1),         # sizes are still checked
    (dict(dt=3), 2),
    (dict(m=-1), 1),
    (dict(nout=-1), 1),
    (dict(eps=math.nan), 1),
    (dict(eps=math.inf), 1),
    (dict(h=None), 1),
    (dict(out=None), 1),
    (dict(m=9), 1),               # more rows than h has, no row_idx
    (dict(h=8), 3),
    (dict(ldo=60), 3),
    (dict(ldh=68), 3),            # 136 bytes: not a multiple of 16
    (dict(gamma=24), 3),
])
def test_exit_projection_argument_errors(kw, status):
    assert _exit_projection(**kw) == status
    if status:
        assert len(tee.load().river_last_error()) > 0


def test_kv_fill_layer_argument_errors():
    lib = tee.load()
    w = tee.RiverW4(16, 16, 16, tee.RIVER_BF16, 64)

    def call(layer, **k):
        a = dict(m=8, mdev=None, d=128, dt=tee.RIVER_BF16, h=16, ld=128, nrows=8, ri=None,
                 slot=16, nl=2, maps=None, wk=ctypes.byref(w), wv=ctypes.byref(w),
                 lay=None if layer is None else ctypes.byref(layer), hk=2, hd=64, kc=16, vc=16,
                 ns=8, ws=None, wsn=0, s=None)
        a.update(k)
        return lib.river_kv_fill_layer(*a.values())

    L = tee.RiverLayer
    assert call(None, m=0) == 0                                         # empty call
    assert call(L(16, 1e-6, None, None, None, None, None, 0)) == 5      # a norm needs a workspace
    assert call(L(16, math.nan, None, None, None, None, None, 0), ws=16, wsn=1 << 30) == 1
    assert call(L(None, 0.0, None, None, 16, None, 16, 64)) == 1        # rotation without cos
    assert call(L(None, 0.0, None, None, 16, 16, 16, 0)) == 1           # empty tables
    assert call(L(None, 0.0, None, None, 16, 16, 16, 64), hd=63, hk=2) == 1   # odd head_dim
    assert call(L(None, 0.0, None, None, 16, 16, 24, 64)) == 3          # misaligned table
    assert call(L(None, 0.0, 8, None, None, None, None, 0)) == 3        # misaligned bias
    need = tee.river_workspace_size(tee.OP_KV_FILL_LAYER, 8, 128, 0, 0, 1)
    assert need >= 8 * 128 * 2 + 2 * 8 * 4
    assert call(L(16, 1e-6, None, None, None, None, None, 0), ws=16, wsn=need - 1) == 5


def test_decode_step_argument_errors():
    lib = tee.load()
    w = tee.RiverW4(16, 16, 16, tee.RIVER_BF16, 64)
    C = tee.RiverCheckpoint

    def call(cks, **k):
        arr = (C * len(cks))(*cks)
        a = dict(n=8, d=128, dt=tee.RIVER_BF16, ld=128, nck=len(cks), ck=arr, L=4, gamma=None,
                 eps=1e-6, b=0, rule=0, wk=ctypes.byref(w), wv=ctypes.byref(w), hk=2, hd=64,
                 slot=16, kc=16, vc=16, ns=8, ex=16, ws=16, wsn=1 << 30, s=None)
        a.update(k)
        return lib.river_decode_step(*a.values())

    ok = C(1, 16, 16, 0.5, -math.inf, None, None, None)
    assert call([ok], n=0) == 0                                          # empty batch
    assert call([C(0, 16, 16, 0.5, 0.0, None, None, None)]) == 1         # layer 0
    assert call([C(4, 16, 16, 0.5, 0.0, None, None, None)]) == 1         # layer L
    assert call([C(2, 16, 16, 0.5, 0.0, None, None, None), ok]) == 1     # decreasing layers
    assert call([C(1, None, 16, 0.5, 0.0, None, None, None)]) == 1       # no states
    assert call([C(1, 16, 16, math.nan, 0.0, None, None, None)]) == 1    # NaN tau
    assert call([C(1, 16, 16, 0.5, 0.0, 16, None, None)], b=8) == 1     # router without w_up
    assert call([C(1, 8, 16, 0.5, 0.0, None, None, None)]) == 3          # misaligned state
    assert call([ok], ws=None, wsn=0) == 5                               # no workspace
    assert call([ok], ex=None) == 1
    assert call([ok], rule=3) == 1
    need = tee.river_workspace_size(tee.OP_DECODE_STEP, 8, 128, 0, 0, 4)
    assert need > 0
    assert call([C(1, 16, 16, 0.5, 0.0, None, None, 16)], wsn=need // 8) == 5   # maps need x_hat


def test_router_fit_argument_errors():
    lib = tee.load()

    def call(**k):
        a = dict(n=64, d=128, dt=tee.RIVER_BF16, h=16, ld=128, y=16, gamma=None, eps=1e-6, b=16,
                 wd=16, wu=16, epochs=2, batch=32, order=None, lr=1e-3, b1=0.9, b2=0.999,
                 aeps=1e-8, loss=None, ws=16, wsn=1 << 30, s=None)
        a.update(k)
        return lib.river_router_fit(*a.values())

    assert call(n=0) == 1
    assert call(epochs=0) == 1
    assert call(b=513) == 1
    assert call(batch=1001) == 1
    assert call(lr=0.0) == 1
    assert call(b1=1.0) == 1
    assert call(aeps=0.0) == 1
    assert call(y=None) == 1
    assert call(h=8) == 3
    assert call(ws=None, wsn=0) == 5
    need = tee.river_workspace_size(tee.OP_ROUTER_FIT, 64, 128, 16, 32, 2)
    assert need >= 3 * 128 * 16 * 4
    assert call(wsn=need - 1) == 5


# ------------------------------------------------- fill chunk and path plan

def test_kv_fill_plan_keeps_room_for_dequantised_weights():
    """A workspace sized for 6 of 12 layers at 4096 rows (d = 1024, n_out =
    1024): the chunk leaves room for its dequantised weights, so the
    projection takes the path the size was meant for, instead of the chunk
    taking that room as x_hat layers and the projection falling back to
    registers."""
    m, d, no = 4096, 1024, 1024
    xb = m * d * 2
    tee.river_debug_set_fill_fuse(1)             # the x_hat path (not through the product)
    try:
        _plan_keeps_room(m, d, no, xb)
    finally:
        tee.river_debug_set_fill_fuse(0)


def _plan_keeps_room(m, d, no, xb):
    ws = tee.river_workspace_size(tee.OP_KV_FILL, m, d, no, 0, 6)
    chunk, path, parts = tee.river_debug_kv_fill_plan(m, d, no, 12, ws)
    assert path == 2 and parts == 1
    assert chunk * xb + chunk * 2 * no * d * 2 <= ws
    assert chunk == 6
    # sized for every layer: one chunk of all of them, dequantised weights
    ws = tee.river_workspace_size(tee.OP_KV_FILL, m, d, no, 0, 12)
    assert tee.river_debug_kv_fill_plan(m, d, no, 12, ws) == (12, 2, 1)
    # x_hat only: fewer layers per chunk, the rest for the weights
    ws = tee.river_workspace_size(tee.OP_KV_FILL, m, d, 0, 0, 6)
    chunk, path, _ = tee.river_debug_kv_fill_plan(m, d, no, 6, ws)
    assert path == 2 and 1 <= chunk < 6 and chunk * xb + chunk * 2 * no * d * 2 <= ws
    # one layer of x_hat and nothing more: in registers
    ws = tee.river_workspace_size(tee.OP_KV_FILL, m, d, 0, 0, 1)
    assert tee.river_debug_kv_fill_plan(m, d, no, 6, ws) == (1, 0, 1)
    # the row count on the device: never dequantised automatically
    ws = tee.river_workspace_size(tee.OP_KV_FILL, m, d, no, 0, 12)
    assert tee.river_debug_kv_fill_plan(m, d, no, 12, ws, dev_count=True) == (12, 0, 1)


@pytest.mark.parametrize("m,d,nl,want,want_xhat", [
    (30704, 5120, 48, (48, 3, 1), (48, 2, 1)),     # long-context prefill at 32K tokens
    (63472, 5120, 48, (48, 3, 1), (48, 2, 1)),     # and at 64K
    (7782, 4096, 1, (1, 3, 1), (1, 2, 1)),         # 8B prefill, the late exits
    (410, 4096, 21, (21, 0, 1), (21, 0, 1)),       # 8B prefill, the early exits
    (64, 4096, 8, (8, 1, 4), (8, 1, 4)),           # decode-sized: split reduction
])
def test_kv_fill_plan_at_the_workload_shapes(m, d, nl, want, want_xhat):
    """From 4 n_out rows given on the host the fill runs through the product
    of weights and maps (path 3); below, and with the row count on the
    device, through x_hat; the fill-fuse hook can switch the product off."""
    ws = tee.river_workspace_size(tee.OP_KV_FILL, m, d, 1024, 0, nl)
    assert tee.river_debug_kv_fill_plan(m, d, 1024, nl, ws) == want
    assert tee.river_debug_kv_fill_plan(m, d, 1024, nl, ws, dev_count=True)[1] != 3
    tee.river_debug_set_fill_fuse(1)
    try:
        assert tee.river_debug_kv_fill_plan(m, d, 1024, nl, ws) == want_xhat
    finally:
        tee.river_debug_set_fill_fuse(0)


def test_kv_fill_plan_product_chunks_by_its_own_layer_size():
    """Through the product a layer needs its dequantised K|V weights, its
    transposed map and the product (2 x 2 n_out d + d^2 bf16), so a
    workspace for fewer layers splits the call into chunks of that many."""
    m, d, no, nl = 63472, 5120, 1024, 48
    per = 2 * (2 * no * d * 2) + d * d * 2
    assert tee.river_debug_kv_fill_plan(m, d, no, nl, 10 * per + 100) == (10, 3, 1)
    tee.river_debug_set_fill_fuse(2)
    try:
        # forced: from one row on, whatever the count, when a layer's room fits
        per = 2 * (2 * 1024 * 1024 * 2) + 1024 * 1024 * 2
        assert tee.river_debug_kv_fill_plan(300, 1024, 1024, 4, 4 * per) == (4, 3, 1)
        assert tee.river_debug_kv_fill_plan(300, 1024, 1024, 4, per - 1)[1] != 3
    finally:
        tee.river_debug_set_fill_fuse(0)


def test_kv_fill_plan_rejects_a_workspace_under_one_layer():
    with pytest.raises(tee.RiverError) as e:
        tee.river_debug_kv_fill_plan(4096, 1024, 1024, 4, 1024)
    assert e.value.name == "ERR_WORKSPACE"


# ------------------------------------------------- 31-bit operand spans

def test_long_context_64k_spans_fit_31_bits():
    """Every byte span the MFMA fill addresses with 32-bit offsets, at the
    long-context shape with 65536 tokens (63,472 filled rows, d = 5120,
    48 layers of 8 x 128 K/V heads), stays below 2^31: the states it
    gathers from, one layer of x_hat, one map, the dequantised K/V weights
    of one layer, and one layer of the cache that the epilogue indexes in
    64-bit; the ridge fit's transposed operands at 16384 calibration
    tokens. The whole caches and the x_hat of all layers are larger, and
    are only ever offset in 64 bits by layer."""
    lim = 1 << 31
    N, m, d, nl, n_out, n_calib = 65536, 63472, 5120, 48, 1024, 16384
    assert N * d * 2 < lim                       # h, gathered rows (map GEMM's A)
    assert m * d * 2 < lim                       # one layer of x_hat (projection's A)
    assert d * d * 2 < lim                       # one map (map GEMM's B)
    assert 2 * n_out * d * 2 < lim               # one layer of dequantised K|V (B)
    assert 4 * n_out * d < lim                   # the span check the fill applies
    assert N * n_out * 2 < lim                   # one cache layer
    assert nl * N * n_out * 2 >= lim             # the whole cache does not: 64-bit layer offsets
    np_ = (n_calib + 255) // 256 * 256
    assert d * np_ * 2 < lim and d * ((3 * d + 255) // 256 * 256) * 2 < lim
    ws = tee.river_workspace_size(tee.OP_KV_FILL, m, d, n_out, 0, nl)
    assert ws >= nl * m * d * 2 + nl * 2 * n_out * d * 2
    # through the product: one layer of F (2 n_out x d, the projection's B)
    # and one transposed map (its B) are the spans above
    assert tee.river_debug_kv_fill_plan(m, d, n_out, nl, ws) == (nl, 3, 1)
    tee.river_debug_set_fill_fuse(1)
    try:
        assert tee.river_debug_kv_fill_plan(m, d, n_out, nl, ws) == (nl, 2, 1)
    finally:
        tee.river_debug_set_fill_fuse(0)


def test_ridge_fit_rejects_31_bit_overflow():
    """A bf16 fit whose transposed operand (d_in x padded n) would need byte
    offsets of 2^31 or more is refused before anything runs."""
    lib = tee.load()
    a = dict(n=210048, d_in=5120, d_out=5120, T=1, X=256, xdt=tee.RIVER_BF16, Y=256,
             ydt=tee.RIVER_BF16, lam=0.1, W=256, wdt=tee.RIVER_BF16, ws=256, wsn=1 << 62, s=None)
    assert lib.river_ridge_fit(*a.values()) == 4
    assert b"2^31" in lib.river_last_error()
    a["n"] = 16384
    a["wsn"] = 0
    assert lib.river_ridge_fit(*a.values()) == 5      # passes the span check, stops at the workspace


# ------------------------------------------------- binding shape checks

def _fill_args(nl=3, n=16, d=256, hk=2, hd=64, slots=32, group=64):
    import torch
    h = torch.zeros(n, d, dtype=torch.bfloat16)
    slot = torch.arange(n, dtype=torch.int32)

    def w(layers=nl):
        return (torch.zeros(layers, hk * hd, d // 2, dtype=torch.uint8),
                torch.ones(layers, hk * hd, d // group, dtype=torch.bfloat16),
                torch.zeros(layers, hk * hd, d // group, dtype=torch.bfloat16), group)
    kc = torch.zeros(nl, slots, hk, hd, dtype=torch.bfloat16)
    return h, slot, w, kc


def test_binding_rejects_mismatched_fill_shapes():
    import torch
    h, slot, w, kc = _fill_args()
    ok = dict(m_max=4)
    with pytest.raises(ValueError, match="wv"):
        tee.river_kv_fill(h, slot, w(), w(2), 2, 64, kc, kc.clone(), **ok)
    with pytest.raises(ValueError, match="k_cache"):
        tee.river_kv_fill(h, slot, w(), w(), 2, 64, kc[:2], kc.clone(), **ok)
    with pytest.raises(ValueError, match="slot count"):
        tee.river_kv_fill(h, slot, w(), w(), 2, 64, kc, kc[:, :16].clone(), **ok)
    with pytest.raises(ValueError, match="slot"):
        tee.river_kv_fill(h, slot[:8], w(), w(), 2, 64, kc, kc.clone(), **ok)
    with pytest.raises(ValueError, match="row_idx"):
        tee.river_kv_fill(h, slot, w(), w(), 2, 64, kc, kc.clone(), m_max=8,
                          row_idx=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="maps"):
        tee.river_kv_fill(h, slot, w(), w(), 2, 64, kc, kc.clone(), m_max=4,
                          maps=torch.zeros(2, 256, 256, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="k_cache"):
        tee.river_kv_fill(h, slot, w(), w(), 4, 32, kc, kc.clone(), **ok)   # heads x dim differ
    with pytest.raises(ValueError, match="k_bias"):
        tee.river_kv_fill_layer(h, slot, w(), w(), 2, 64, kc, kc.clone(), m_max=4,
                                k_bias=torch.zeros(2, 128, dtype=torch.bfloat16))


def test_binding_rejects_mismatched_folded_shapes():
    """The folded fill's wrappers check F, the caches and the dtypes
    against each other before any call (CPU tensors: nothing runs)."""
    import torch
    d, hk, hd, nl = 256, 2, 64, 3
    n_out = hk * hd
    q = torch.zeros((nl, n_out, d // 2), dtype=torch.uint8)
    sz = torch.ones((nl, n_out, d // 64), dtype=torch.bfloat16)
    w = (q, sz, sz, 64)
    F = torch.zeros((nl, 2 * n_out, d), dtype=torch.bfloat16)
    h = torch.zeros((8, d), dtype=torch.bfloat16)
    slot = torch.arange(8, dtype=torch.int32)
    kc = torch.zeros((nl, 16, hk, hd), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tee.river_kv_fold(w, w, hk, hd, F[:, :n_out])                       # F rows != 2 n_out
    with pytest.raises(ValueError):
        tee.river_kv_fold(w, w, hk, hd, F.float())                          # F not bf16
    with pytest.raises(ValueError):
        tee.river_kv_fold(w, w, hk, hd, F, maps=torch.zeros((nl, d, d - 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        tee.river_kv_fill_folded(h, slot, F, hk, hd, kc[:2], kc)            # cache layers != F layers
    with pytest.raises(ValueError):
        tee.river_kv_fill_folded(h.float(), slot, F, hk, hd, kc, kc)        # states not bf16
    with pytest.raises(ValueError):
        tee.river_kv_fill_folded(h, slot[:4], F, hk, hd, kc, kc)            # slot shorter than h


def test_binding_rejects_mismatched_decode_and_ridge_shapes():
    import torch
    h, slot, w, kc = _fill_args(nl=4)
    ck = [{"layer": 1, "h_prev": h, "h_cur": h, "tau": 0.5, "theta": -math.inf}]
    ex = torch.zeros(16, dtype=torch.int32)
    with pytest.raises(ValueError, match="wk"):
        tee.river_decode_step(ck, w(3), w(4), 2, 64, slot, kc, kc.clone(), ex)
    with pytest.raises(ValueError, match="v_cache"):
        tee.river_decode_step(ck, w(4), w(4), 2, 64, slot, kc, kc[:3].clone(), ex)
    with pytest.raises(ValueError, match="maps"):
        ck2 = [dict(ck[0], maps=torch.zeros(4, 256, 256, dtype=torch.bfloat16))]
        tee.river_decode_step(ck2, w(4), w(4), 2, 64, slot, kc, kc.clone(), ex)
    X = torch.zeros(64, 128, dtype=torch.bfloat16)
    Y = torch.zeros(2, 32, 64, dtype=torch.bfloat16)
    W = torch.zeros(2, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="calibration token"):
        tee.river_ridge_fit(X, Y, 0.1, W)
    with pytest.raises(ValueError, match="W must be"):
        tee.river_ridge_fit(X, torch.zeros(2, 64, 64, dtype=torch.bfloat16), 0.1, W[:1])


def test_binding_rejects_mismatched_route_and_compact_shapes():
    import torch
    h = torch.zeros(16, 256, dtype=torch.bfloat16)
    mask = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="h_prev"):
        tee.river_route(h[:8], h, mask)
    with pytest.raises(ValueError, match="w_up"):
        tee.river_route(h, h, mask, w_down=torch.zeros(8, 256, dtype=torch.bfloat16),
                        w_up=torch.zeros(4, dtype=torch.bfloat16))
    i32 = lambda k: torch.zeros(k, dtype=torch.int32)
    with pytest.raises(ValueError, match="exit_idx"):
        tee.river_compact(mask, h, i32(16), i32(8), i32(2))
    with pytest.raises(ValueError, match="out must have"):
        tee.river_compact(mask, h, i32(16), i32(16), i32(2),
                          out=torch.zeros(16, 128, dtype=torch.bfloat16))
