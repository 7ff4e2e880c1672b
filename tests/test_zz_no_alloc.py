"""river_decode_step_static (the decode step on the library's static device
scratch, for callers that cannot allocate) against river_decode_step with a
workspace of the size the static call uses: exit layers and caches equal
bit for bit (the same kernels on the same sizes), on two calls in a row,
the second with fewer tokens; the exits also within the oracle's bar on the
first call. A call whose least workspace exceeds the 64 MiB scratch is
refused with RIVER_ERR_WORKSPACE before anything runs."""

import math

import numpy as np
import pytest
import torch

import bench as B
import oracle as O
import token_early_exit_amd as tee
from synth import get_config
from synth import generate as G
from helpers import f32, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"
INF = math.inf
SCRATCH = 64 << 20


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    tee.river_debug_set_decode_path(0)
    tee.river_debug_set_gemm_path(0)
    yield


def _kv(cfg, layers):
    w = G.kv_weights(cfg, layers, device=DEV)
    return (tuple(w["wk"]) + (cfg.group,), tuple(w["wv"]) + (cfg.group,))


def both(cks, cfg, wk, wv, slot):
    """(exit layers, K, V) of the static call and of river_decode_step with a
    workspace of min(64 MiB, the size for one pass) bytes, each on fresh
    NaN-filled caches."""
    n, d = cks[0]["h_cur"].shape
    n_out = cfg.n_kv_heads * cfg.head_dim
    want = tee.river_workspace_size(tee.OP_DECODE_STEP, n, d, n_out, 0, cfg.L)
    ws = torch.empty(min(want, SCRATCH), dtype=torch.uint8, device=DEV)
    out = []
    for static in (True, False):
        kc, vc = G.nan_cache(cfg, cfg.L, device=DEV)
        ex = torch.full((n,), -7, dtype=torch.int32, device=DEV)
        if static:
            tee.river_decode_step_static(cks, wk, wv, cfg.n_kv_heads, cfg.head_dim, slot, kc, vc, ex)
        else:
            tee.river_decode_step(cks, wk, wv, cfg.n_kv_heads, cfg.head_dim, slot, kc, vc, ex, workspace=ws)
        torch.cuda.synchronize()
        out.append((ex, kc, vc))
    return out, want


def assert_same(a, b):
    (e0, k0, v0), (e1, k1, v1) = a, b
    assert torch.equal(e0, e1)
    assert torch.equal(k0.view(torch.int16), k1.view(torch.int16))
    assert torch.equal(v0.view(torch.int16), v1.view(torch.int16))


def oracle_exits(cks, L):
    """The oracle's exit layer of every token (router off)."""
    n = cks[0]["h_cur"].shape[0]
    ex = np.full(n, L)
    alive = np.ones(n, bool)
    band = np.zeros(n, bool)
    for c in cks:
        cos, _, m, _ = O.route(np64(c["h_prev"]), np64(c["h_cur"]), None, 1e-6, None, None,
                               f32(c["tau"]), -INF)
        band |= alive & (np.abs(cos - f32(c["tau"])) < 1e-4)
        dec = (m != 0) & alive
        ex[dec] = c["layer"]
        alive &= ~dec
    return ex, band


def llama1b(n, tag="eval"):
    cfg = get_config(2, n_tokens=n)
    hs = {l: t.to(DEV) for l, t in G.hidden_states(cfg, n, range(7, 17), tag=tag).items()}
    alive = np.ones(n, bool)
    cks = []
    for l in cfg.route_layers:
        cos, *_ = O.route(np64(hs[l - 1]), np64(hs[l]), None, 1e-6, None, None, -INF, -INF)
        c = np.sort(cos[alive])
        m = len(c)
        tau = 0.5 * (c[(m - 1) // 2] + c[m // 2]) if m > 1 else (c[0] - 1 if m else 0.0)
        cks.append({"layer": l, "h_prev": hs[l - 1], "h_cur": hs[l], "tau": tau, "theta": -INF})
        alive &= ~(cos > f32(tau))
    return cfg, cks


def test_static_decode_llama1b_two_calls():
    """Llama-3.2-1B decode (router off, identity fill): 64 tokens, then 37."""
    cfg, cks = llama1b(64)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    (a, b), want = both(cks, cfg, wk, wv, slot)
    assert want <= SCRATCH                       # the whole step fits: one pass, split reductions
    assert_same(a, b)
    ex_ref, band = oracle_exits(cks, cfg.L)
    assert np.array_equal(a[0].cpu().numpy()[~band], ex_ref[~band])
    assert (a[0] < cfg.L).any()
    # second call, fewer tokens (other states): the scratch keeps the first
    # call's contents, which must not leak into the result
    cfg2, cks2 = llama1b(37, tag="second")
    slot2 = G.slots(cfg2, n=37, device=DEV)
    (a2, b2), _ = both(cks2, cfg2, wk, wv, slot2)
    assert_same(a2, b2)
    ex2, band2 = oracle_exits(cks2, cfg2.L)
    assert np.array_equal(a2[0].cpu().numpy()[~band2], ex2[~band2])


def llama8b(n, tag="eval"):
    cfg = get_config("3D", n_tokens=n)
    layers = list(cfg.route_layers)
    need = sorted({l - 1 for l in layers} | set(layers))
    hs = G.hidden_states(cfg, n, need, tag=tag, device=DEV)
    cks = []
    for l in layers:
        wd, wu = G.router_weights(cfg, l, device=DEV)
        c = {"layer": l, "h_prev": hs[l - 1], "h_cur": hs[l], "tau": -INF, "theta": INF,
             "w_down": wd, "w_up": wu}
        if l == 11:
            _, prob, _, _ = O.route(np64(hs[10]), np64(hs[11]), None, 1e-6, np64(wd), np64(wu), -INF, -INF)
            p = np.sort(prob)[::-1]
            k = max(1, n // 20)
            c["theta"] = 0.5 * (p[k - 1] + p[k])
            c["maps"] = G.near_identity_maps(cfg, cfg.L - l, device=DEV)
        if l == 31:
            c["theta"] = -INF
            c["maps"] = G.near_identity_maps(cfg, cfg.L - l, tag="maps31", device=DEV)
        cks.append(c)
    return cfg, cks


def test_static_decode_8b_routers_maps_two_calls():
    """Llama-3-8B decode (routers at every fourth block, maps at 11 and 31):
    256 tokens, whose full workspace is larger than the scratch (the fills
    run in chunks of layers), then 100 tokens."""
    cfg, cks = llama8b(256)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    (a, b), want = both(cks, cfg, wk, wv, slot)
    assert want > SCRATCH
    assert_same(a, b)
    e = a[0].cpu().numpy()
    assert (e == 11).sum() >= 10 and (e == 31).sum() + (e == 11).sum() == 256
    cfg2, cks2 = llama8b(100, tag="second")
    slot2 = G.slots(cfg2, n=100, device=DEV)
    (a2, b2), _ = both(cks2, cfg2, wk, wv, slot2)
    assert_same(a2, b2)


def test_static_decode_8b_folded_two_calls():
    """The same step with the maps folded into the K/V weights beforehand
    (river_kv_fold: those checkpoints fill without workspace), then 100
    tokens."""
    cfg, cks = llama8b(256)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    B.fold_checkpoints(cfg, cks, wk, wv, DEV)
    (a, b), _ = both(cks, cfg, wk, wv, slot)
    assert_same(a, b)
    e = a[0].cpu().numpy()
    assert (e == 11).sum() >= 10 and (e == 31).sum() + (e == 11).sum() == 256
    cfg2, cks2 = llama8b(100, tag="second")
    B.fold_checkpoints(cfg2, cks2, wk, wv, DEV)
    slot2 = G.slots(cfg2, n=100, device=DEV)
    (a2, b2), _ = both(cks2, cfg2, wk, wv, slot2)
    assert_same(a2, b2)


def test_static_decode_refuses_more_than_the_scratch():
    """4096 tokens of d = 8192: the step's fixed scratch alone exceeds 64 MiB."""
    n, d, L = 4096, 8192, 4
    h = torch.zeros(n, d, dtype=torch.bfloat16, device=DEV)
    w = (torch.zeros(L, 128, d // 2, dtype=torch.uint8, device=DEV),
         torch.ones(L, 128, d // 128, dtype=torch.bfloat16, device=DEV),
         torch.zeros(L, 128, d // 128, dtype=torch.bfloat16, device=DEV), 128)
    kc = torch.zeros(L, n, 1, 128, dtype=torch.bfloat16, device=DEV)
    ex = torch.zeros(n, dtype=torch.int32, device=DEV)
    slot = torch.arange(n, dtype=torch.int32, device=DEV)
    cks = [{"layer": 1, "h_prev": h, "h_cur": h, "tau": 0.5, "theta": -INF}]
    with pytest.raises(tee.RiverError) as err:
        tee.river_decode_step_static(cks, w, w, 1, 128, slot, kc, kc.clone(), ex)
    assert err.value.name == "ERR_WORKSPACE" and "static scratch" in str(err.value)
    assert bool((ex == 0).all())
