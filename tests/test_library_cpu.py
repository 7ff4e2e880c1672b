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


def test_workspace_sizes():
    ws = tee.river_workspace_size
    assert ws(tee.OP_ROUTE, 4096, 768) == 0
    assert ws(tee.OP_KV_FILL, 4096, 768, 0, 0, 0) == 0           # identity: none
    assert ws(tee.OP_KV_FILL, 4096, 768, 0, 0, 8) >= 8 * 4096 * 768 * 2
    assert ws(tee.OP_COMPACT, 100000) >= 4 * 25
    assert ws(tee.OP_RIDGE_FIT, 2048, 768, 768, 8, tee.RIVER_BF16) > 0
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
    assert lib.river_debug_set_gemm_path(3) == 1
    assert lib.river_debug_set_decode_path(2) == 1


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
