"""GPU parity: the HIP library (through its C interface) against the float64
oracle on the same seeded inputs.

Bars: masks and indices bit-exact (tokens within 1e-4 of a threshold are
excluded and counted); |d cos|, |d prob| <= 2e-3; K/V per-row relative L2
error <= 1e-2 against the oracle on the same int4 weights and bf16 maps;
ridge maps within 1e-3 (fp32 out) or 5e-3 (bf16 out) relative Frobenius.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import token_early_exit_amd as tee
from synth import get_config
from synth import generate as G
from helpers import (BAND, KV_TOL, check_route, f32, kv_row_errors, midpoint_threshold, np64,
                     w4_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"
INF = math.inf


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    tee.river_debug_set_compact_path(0)
    yield
    tee.river_debug_set_compact_path(0)


# ------------------------------------------------------------------ route

def route_gpu(hp, hc, wd, wu, tau, theta, rule=O.RULE_TOKEN, gamma=None, eps=1e-6):
    n = hc.shape[0]
    cos = torch.full((n,), 7.0, device=DEV)
    prob = torch.full((n,), 7.0, device=DEV)
    mask = torch.full((n,), 9, dtype=torch.uint8, device=DEV)
    alle = torch.full((1,), 9, dtype=torch.int32, device=DEV)
    tee.river_route(hp, hc, mask, gamma=gamma, eps=eps, w_down=wd, w_up=wu, tau=tau, theta=theta,
                    rule=rule, cos_out=cos, prob_out=prob, all_exit_out=alle)
    torch.cuda.synchronize()
    return cos, prob, mask, alle[0]


def route_ref(hp, hc, wd, wu, tau, theta, rule=O.RULE_TOKEN, gamma=None, eps=1e-6):
    return O.route(np64(hp), np64(hc), None if gamma is None else np64(gamma), eps,
                   None if wd is None else np64(wd), None if wu is None else np64(wu),
                   f32(tau), f32(theta), rule)


def _states(cfg, n, layers, device=DEV):
    return {l: t.to(device) for l, t in G.hidden_states(cfg, n, layers, device="cpu").items()}


@pytest.mark.parametrize("layer", [2, 4, 6])
@pytest.mark.parametrize("rule", [O.RULE_TOKEN, O.RULE_BATCH_MIN])
def test_route_tiny_fp32(layer, rule):
    cfg = get_config(0)
    hs = _states(cfg, cfg.n_tokens, [layer - 1, layer])
    wd, wu = (t.to(DEV) for t in G.router_weights(cfg, layer))
    args = (hs[layer - 1], hs[layer], wd, wu, cfg.tau, cfg.theta, rule)
    excl = check_route(route_gpu(*args), route_ref(*args), cfg.tau, cfg.theta, True, rule)
    assert excl <= 1


@pytest.mark.parametrize("n", [4096, 4091, 17, 1])
def test_route_gpt2_prefill(n):
    cfg = get_config(1)
    hs = _states(cfg, cfg.n_tokens, [3, 4])
    wd, wu = (t.to(DEV) for t in G.router_weights(cfg, 4))
    args = (hs[3][:n], hs[4][:n], wd, wu, cfg.tau, cfg.theta)
    gpu = route_gpu(*args)
    excl = check_route(gpu, route_ref(*args), cfg.tau, cfg.theta, True)
    assert excl <= max(1, n // 100)
    if n == 4096:
        frac = gpu[2].float().mean().item()
        assert 0.05 < frac < 0.95        # the router splits the batch (13% exit at seed 0)


def test_route_8b_shape_two_row_tiles():
    cfg = get_config(3)
    hs = {l: t for l, t in G.hidden_states(cfg, 8192, [10, 11], device=DEV).items()}
    wd, wu = G.router_weights(cfg, 11, device=DEV)
    _, prob, _, _ = route_ref(hs[10], hs[11], wd, wu, -INF, -INF)
    theta = midpoint_threshold(prob, 410)          # ~5% exit at this checkpoint
    args = (hs[10], hs[11], wd, wu, -INF, theta)
    gpu = route_gpu(*args)
    excl = check_route(gpu, route_ref(*args), -INF, theta, True)
    assert excl <= 82
    assert abs(int(gpu[2].sum()) - 410) <= excl + 1


def test_route_with_gamma_and_odd_width():
    g = torch.Generator().manual_seed(5)
    n, d, b = 300, 512, 96
    hp = torch.randn(n, d, generator=g).bfloat16().to(DEV)
    hc = (hp.float().cpu() + 0.3 * torch.randn(n, d, generator=g)).bfloat16().to(DEV)
    gamma = (0.5 + torch.rand(d, generator=g)).bfloat16().to(DEV)
    wd = (torch.randn(b, d, generator=g) / d ** 0.5).bfloat16().to(DEV)
    wu = (torch.randn(b, generator=g) / b ** 0.5).bfloat16().to(DEV)
    args = (hp, hc, wd, wu, 0.5, 0.5)
    check_route(route_gpu(*args, gamma=gamma), route_ref(*args, gamma=gamma), 0.5, 0.5, True)


@pytest.mark.parametrize("n", [8192, 8195])
def test_route_large_batch_gamma_narrow_router(n):
    """32-token workgroups (from 8192 tokens) with gamma, a router of 64
    units (half the waves own none) and a ragged last workgroup."""
    g = torch.Generator().manual_seed(n)
    d, b = 1024, 64
    hp = torch.randn(n, d, generator=g).bfloat16().to(DEV)
    hc = (hp.float().cpu() + 0.3 * torch.randn(n, d, generator=g)).bfloat16().to(DEV)
    gamma = (0.5 + torch.rand(d, generator=g)).bfloat16().to(DEV)
    wd = (torch.randn(b, d, generator=g) / d ** 0.5).bfloat16().to(DEV)
    wu = (torch.randn(b, generator=g) / b ** 0.5).bfloat16().to(DEV)
    args = (hp, hc, wd, wu, 0.5, 0.5)
    check_route(route_gpu(*args, gamma=gamma), route_ref(*args, gamma=gamma), 0.5, 0.5, True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_route_edges(dtype):
    g = torch.Generator().manual_seed(6)
    d = 256
    a = torch.randn(8, d, generator=g)
    hp = a.clone()
    hc = a.clone()
    hc[1] = -a[1]                    # cos = -1
    hc[2] = 3.0 * a[2]               # cos = 1
    hp[3] = 0.0                      # zero norm: cos = 0
    hp[4, 7] = float("nan")          # NaN: never exits
    hc[5] = a[5] + 0.5 * torch.randn(d, generator=g)
    hp, hc = hp.to(dtype).to(DEV), hc.to(dtype).to(DEV)
    wd = (torch.randn(32, d, generator=g) / 16).to(dtype).to(DEV)
    wu = torch.randn(32, generator=g).to(dtype).to(DEV)
    for router in (False, True):
        w = (wd, wu) if router else (None, None)
        cos, prob, mask, alle = route_gpu(hp, hc, *w, -INF, -INF)
        c = cos.cpu().numpy()
        assert abs(c[0] - 1) <= 2e-3 and abs(c[1] + 1) <= 2e-3 and abs(c[2] - 1) <= 2e-3
        assert c[3] == 0.0 and np.isnan(c[4]) and mask[4].item() == 0
        assert int(alle) == 0
        check_route((cos, prob, mask, alle), route_ref(hp, hc, *w, -INF, -INF), -INF, -INF, router)
    # empty batch: all_exit is 0
    z = torch.empty(0, d, dtype=dtype, device=DEV)
    _, _, _, alle = route_gpu(z, z, wd, wu, 0.0, 0.0, O.RULE_BATCH_MIN)
    assert int(alle) == 0
    # zero router weights: prob is exactly 1/2 and theta = 1/2 lets nobody exit
    _, prob, mask, _ = route_gpu(hp, hc, torch.zeros_like(wd), wu, -INF, 0.5)
    assert torch.all(prob == 0.5) and int(mask.sum()) == 0


def test_route_router_off_decode_shape():
    cfg = get_config(2)
    hs = _states(cfg, cfg.n_tokens, [7, 8])
    c, *_ = route_ref(hs[7], hs[8], None, None, -INF, -INF)
    tau = 0.5 * (np.sort(c)[31] + np.sort(c)[32])
    for rule in (O.RULE_TOKEN, O.RULE_BATCH_MIN):
        args = (hs[7], hs[8], None, None, tau, -INF, rule)
        check_route(route_gpu(*args), route_ref(*args), tau, -INF, False, rule)


# ---------------------------------------------------------------- compact

def compact_gpu(mask, h, row_ids=None, out=None):
    n = mask.shape[0]
    d = h.shape[1]
    cont = torch.full((n,), -5, dtype=torch.int32, device=DEV)
    ext = torch.full((n,), -5, dtype=torch.int32, device=DEV)
    counts = torch.full((2,), -5, dtype=torch.int32, device=DEV)
    hc = torch.full_like(h, float("nan"))
    ridc = torch.full((n,), -5, dtype=torch.int32, device=DEV)
    ws = torch.zeros(max(tee.river_workspace_size(tee.OP_COMPACT, n), 16), dtype=torch.uint8,
                     device=DEV)
    tee.river_compact(mask, h, cont, ext, counts, row_ids=row_ids, h_cont=hc, row_ids_cont=ridc,
                      out=out, workspace=ws)
    torch.cuda.synchronize()
    return cont, ext, counts, hc, ridc


@pytest.mark.parametrize("path", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("n", [0, 1, 33, 63, 64, 65, 1023, 1024, 1025, 5000, 8192, 8193, 20000])
def test_compact_all_paths(path, n):
    if path == 1 and n > 64:
        pytest.skip("the ballot path takes n <= 64")
    tee.river_debug_set_compact_path(path)
    g = torch.Generator().manual_seed(n + 17 * path)
    d = 64
    h = torch.randn(n, d, generator=g).bfloat16().to(DEV)
    rid = torch.randperm(2 * n + 3, generator=g)[:n].to(torch.int32).to(DEV)
    for kind in ("random", "zeros", "ones", "sparse"):
        if kind == "random":
            m = (torch.rand(n, generator=g) < 0.5)
        elif kind == "zeros":
            m = torch.zeros(n, dtype=torch.bool)
        elif kind == "ones":
            m = torch.ones(n, dtype=torch.bool)
        else:
            m = torch.rand(n, generator=g) < 0.01
        mask = (m.to(torch.uint8) * torch.randint(1, 255, (n,), generator=g, dtype=torch.uint8)).to(DEV)
        out = torch.full((2 * n + 3, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        cont, ext, counts, hc, ridc = compact_gpu(mask, h, rid, out)
        ref = O.compact(mask.cpu().numpy(), h.cpu().float().numpy(), rid.cpu().numpy(),
                        out.cpu().float().numpy())
        nc, ne = (int(x) for x in ref["counts"])
        assert counts.cpu().tolist() == [nc, ne]
        assert np.array_equal(cont.cpu().numpy()[:nc], ref["cont_idx"])
        assert np.array_equal(ext.cpu().numpy()[:ne], ref["exit_idx"])
        assert np.all(cont.cpu().numpy()[nc:] == -5) and np.all(ext.cpu().numpy()[ne:] == -5)
        assert np.array_equal(ridc.cpu().numpy()[:nc], ref["row_ids_cont"])
        # rows are copies: bitwise equal
        assert torch.equal(hc[:nc].view(torch.int16), h[torch.from_numpy(ref["cont_idx"]).to(DEV)].view(torch.int16))
        o = out.cpu().float().numpy()
        assert np.array_equal(np.isnan(o), np.isnan(ref["out"]))
        assert np.array_equal(np.nan_to_num(o), np.nan_to_num(ref["out"]))
        # deterministic
        again = compact_gpu(mask, h, rid, None)
        assert torch.equal(again[0][:nc], cont[:nc]) and torch.equal(again[1][:ne], ext[:ne])


@pytest.mark.parametrize("n", [4096, 16385])
@pytest.mark.parametrize("d,dt", [(8, torch.bfloat16), (72, torch.bfloat16), (768, torch.bfloat16),
                                  (4096, torch.bfloat16), (1000, torch.float32)])
def test_compact_fused_row_lengths(n, d, dt):
    """The fused launch (16 tokens per workgroup up to 16384 tokens, 64
    beyond) on rows of one 16-byte piece, a ragged number of pieces, and
    rows needing several passes, with gathered continuing rows and
    scattered exits, against the oracle."""
    tee.river_debug_set_compact_path(0)
    g = torch.Generator().manual_seed(n + d)
    h = torch.randn(n, d, generator=g).to(dt).to(DEV)
    rid = torch.randperm(n + 5, generator=g)[:n].to(torch.int32).to(DEV)
    m = torch.rand(n, generator=g) < 0.13
    mask = m.to(torch.uint8).to(DEV)
    out = torch.full((n + 5, d), float("nan"), dtype=dt, device=DEV)
    cont, ext, counts, hc, ridc = compact_gpu(mask, h, rid, out)
    ref = O.compact(mask.cpu().numpy(), h.cpu().float().numpy(), rid.cpu().numpy(),
                    out.cpu().float().numpy())
    nc, ne = (int(x) for x in ref["counts"])
    assert counts.cpu().tolist() == [nc, ne]
    assert np.array_equal(cont.cpu().numpy()[:nc], ref["cont_idx"])
    assert np.array_equal(ext.cpu().numpy()[:ne], ref["exit_idx"])
    iv = torch.int16 if dt == torch.bfloat16 else torch.int32
    assert torch.equal(hc[:nc].view(iv), h[torch.from_numpy(ref["cont_idx"]).to(DEV)].view(iv))
    o = out.cpu().float().numpy()
    assert np.array_equal(np.isnan(o), np.isnan(ref["out"]))
    assert np.array_equal(np.nan_to_num(o), np.nan_to_num(ref["out"]))


def test_compact_row_id_out_of_range_is_skipped():
    n, d = 10, 64
    h = torch.randn(n, d).bfloat16().to(DEV)
    rid = torch.tensor([0, 1, 2, 3, 4, 5, 6, 7, 100, -3], dtype=torch.int32, device=DEV)
    mask = torch.ones(n, dtype=torch.uint8, device=DEV)
    out = torch.zeros(12, d, dtype=torch.bfloat16, device=DEV)
    compact_gpu(mask, h, rid, out)
    assert torch.equal(out[:8], h[:8]) and torch.all(out[8:] == 0)


# ---------------------------------------------------------------- kv_fill

def _kv(cfg, layers, device=DEV):
    w = G.kv_weights(cfg, layers, device="cpu" if device == DEV and cfg.d <= 2048 else device)
    wk = tuple(t.to(DEV) for t in w["wk"]) + (cfg.group,)
    wv = tuple(t.to(DEV) for t in w["wv"]) + (cfg.group,)
    return wk, wv


def fill_gpu(cfg, h, slot, wk, wv, n_layers, row_idx=None, m_dev=None, m_max=None, maps=None,
             ws_layers=None, caches=None):
    kc, vc = caches if caches is not None else G.nan_cache(cfg, n_layers, device=DEV)
    mm = m_max if m_max is not None else (row_idx.shape[0] if row_idx is not None else h.shape[0])
    ws = None
    if maps is not None:
        nl = n_layers if ws_layers is None else ws_layers
        ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, mm, cfg.d, 0, 0, nl),
                         dtype=torch.uint8, device=DEV)
    tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=mm,
                      m_dev=m_dev, row_idx=row_idx, maps=maps, workspace=ws)
    torch.cuda.synchronize()
    return kc, vc


def check_fill(cfg, kc, vc, h, rows, slot, maps, wk, wv, sample=None):
    """Compare filled slots with the oracle; untouched slots must stay NaN."""
    rows = np.asarray(rows)
    slot_np = slot.cpu().numpy()
    pick = np.arange(len(rows)) if sample is None else sample
    # float32 copies hold the bf16 / fp32 values exactly; the oracle widens per layer
    K, V = O.kv_fill_rows(h.float().cpu().numpy(), rows[pick], len(pick),
                          None if maps is None else maps.float().cpu().numpy(), w4_np(wk), w4_np(wv))
    s = torch.from_numpy(slot_np[rows[pick]].astype(np.int64)).to(DEV)
    gk = kc[:, s].reshape(kc.shape[0], len(pick), -1)
    gv = vc[:, s].reshape(vc.shape[0], len(pick), -1)
    ek = kv_row_errors(gk, K)
    ev = kv_row_errors(gv, V)
    assert ek.max() <= KV_TOL and ev.max() <= KV_TOL, (ek.max(), ev.max())
    # exactly the filled slots changed
    filled = torch.zeros(kc.shape[1], dtype=torch.bool)
    filled[torch.from_numpy(slot_np[rows].astype(np.int64))] = True
    nan_k = torch.isnan(kc).all(dim=-1).all(dim=-1).cpu()
    assert torch.all(nan_k[:, ~filled]) and not torch.any(nan_k[:, filled])
    return ek.max(), ev.max()


def test_kv_fill_tiny_fp32_with_ridge_maps():
    cfg = get_config(0)
    e = 2
    layers = list(range(e + 1, cfg.L + 1))
    X, Y = G.calibration(cfg, e)
    maps = torch.from_numpy(O.ridge_fit(np64(X), np64(Y), cfg.ridge_lambda)).float().to(DEV)
    h = G.hidden_states(cfg, cfg.n_tokens, [e])[e].to(DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers)
    rows = torch.tensor([0, 5, 9, 31, 63, 2], dtype=torch.int32, device=DEV)
    kc, vc = fill_gpu(cfg, h, slot, wk, wv, len(layers), row_idx=rows, maps=maps)
    check_fill(cfg, kc, vc, h, rows.cpu().numpy(), slot, maps, wk, wv)


@pytest.mark.parametrize("ws_layers", [8, 3, 1])
def test_kv_fill_gpt2_ridge_maps_device_count(ws_layers):
    cfg = get_config(1)
    e = 4
    layers = list(range(e + 1, cfg.L + 1))
    X, Y = G.calibration(cfg, e)
    maps = torch.from_numpy(O.ridge_fit(np64(X), np64(Y), cfg.ridge_lambda)).bfloat16().to(DEV)
    h = G.hidden_states(cfg, cfg.n_tokens, [e])[e].to(DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers)
    g = torch.Generator().manual_seed(3)
    sel = torch.nonzero(torch.rand(cfg.n_tokens, generator=g) < 0.5).flatten().to(torch.int32)
    rows = torch.full((cfg.n_tokens,), -1, dtype=torch.int32)
    rows[: sel.numel()] = sel
    rows = rows.to(DEV)
    m_dev = torch.tensor([sel.numel()], dtype=torch.int32, device=DEV)
    kc, vc = fill_gpu(cfg, h, slot, wk, wv, len(layers), row_idx=rows, m_dev=m_dev,
                      m_max=cfg.n_tokens, maps=maps, ws_layers=ws_layers)
    pick = np.random.default_rng(0).choice(sel.numel(), 256, replace=False)
    check_fill(cfg, kc, vc, h, sel.numpy(), slot, maps, wk, wv, sample=np.sort(pick))


@pytest.mark.parametrize("gemm_path", [1, 2])
def test_kv_fill_map_gemm_tiles(gemm_path):
    """The map GEMM on 128 x 128 and on 256 x 256 tiles (forced), d = 1024,
    three layers, 300 of 640 rows (a ragged last row tile in both) with the
    count on the device: every filled row within the K/V bar, the two tiles
    within bf16 rounding of each other."""
    cfg = get_config(1, d=1024, n_tokens=640, n_slots=700)
    layers = [5, 6, 7]
    h = G.hidden_states(cfg, cfg.n_tokens, [4])[4].to(DEV)
    g = torch.Generator().manual_seed(1024)
    slot = torch.randperm(cfg.n_slots, generator=g)[: cfg.n_tokens].to(torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, len(layers)).to(DEV)
    sel = torch.sort(torch.randperm(cfg.n_tokens, generator=g)[:300]).values.to(torch.int32)
    rows = torch.full((cfg.n_tokens,), -1, dtype=torch.int32)
    rows[:300] = sel
    m_dev = torch.tensor([300], dtype=torch.int32, device=DEV)
    out = {}
    try:
        for p in (gemm_path, 3 - gemm_path):
            tee.river_debug_set_gemm_path(p)
            out[p] = fill_gpu(cfg, h, slot, wk, wv, len(layers), row_idx=rows.to(DEV), m_dev=m_dev,
                              m_max=cfg.n_tokens, maps=maps)
    finally:
        tee.river_debug_set_gemm_path(0)
    kc, vc = out[gemm_path]
    check_fill(cfg, kc, vc, h, sel.numpy(), slot, maps, wk, wv)
    s = slot[sel.long().to(DEV)].long()
    for a, b in zip(out[1], out[2]):
        a, b = a[:, s].float(), b[:, s].float()
        assert torch.all((a - b).abs() <= 2 ** -6 * b.abs() + 1e-2 * b.abs().amax(dim=-1, keepdim=True))


@pytest.mark.parametrize("nl", [6, 1])
@pytest.mark.parametrize("count", ["device", "host"])
def test_kv_fill_map_narrow_tiles_equal_128_tiles(count, nl):
    """A row bound of at most 256 (a decode step's exits) runs the map GEMM
    on 32-row tiles with an 8-slab ring (automatic). Over several maps each
    tile starts its reduction at its own slab (tiles that run at the same
    time then read different parts of the maps' rows), so its sums run in
    another order than the 128-row tiles' (gemm path 1): the caches agree to
    a few bf16 ulps; over one map they agree bit for bit. Every filled row is
    within the K/V bar. d = 2048, six layers or one; 13 rows under a bound of
    256 with the count on the device, or 200 rows (ragged 32-row tiles) with
    the count on the host."""
    cfg = get_config(1, d=2048, n_tokens=256, n_slots=300)
    layers = [3, 4, 5, 6, 7, 8][:nl]
    h = G.hidden_states(cfg, cfg.n_tokens, [2])[2].to(DEV)
    g = torch.Generator().manual_seed(2048)
    slot = torch.randperm(cfg.n_slots, generator=g)[: cfg.n_tokens].to(torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, len(layers), scale=0.5).to(DEV)
    if count == "device":
        sel = torch.sort(torch.randperm(cfg.n_tokens, generator=g)[:13]).values.to(torch.int32)
        rows = torch.full((cfg.n_tokens,), -1, dtype=torch.int32)
        rows[:13] = sel
        m_max, m_dev = cfg.n_tokens, torch.tensor([13], dtype=torch.int32, device=DEV)
    else:
        sel = torch.sort(torch.randperm(cfg.n_tokens, generator=g)[:200]).values.to(torch.int32)
        rows, m_max, m_dev = sel, 200, None
    out = {}
    try:
        for p in (0, 1):
            tee.river_debug_set_gemm_path(p)
            out[p] = fill_gpu(cfg, h, slot, wk, wv, len(layers), row_idx=rows.to(DEV), m_dev=m_dev,
                              m_max=m_max, maps=maps)
    finally:
        tee.river_debug_set_gemm_path(0)
    s = slot[sel.long().to(DEV)].long()
    for a, b in zip(out[0], out[1]):
        if nl == 1:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        a, b = a[:, s].float(), b[:, s].float()
        assert torch.all((a - b).abs() <= 2 ** -6 * b.abs() + 1e-3 * b.abs().amax(dim=-1, keepdim=True))
    kc, vc = out[0]
    check_fill(cfg, kc, vc, h, sel.numpy(), slot, maps, wk, wv)


@pytest.mark.parametrize("maps", [False, True])
def test_kv_fill_dequantised_projection(maps):
    """The projection as a 256 x 256 bf16 GEMM on weights dequantised into
    the workspace (forced; at large row counts it is the automatic choice),
    d = 1024, 300 of 640 rows with the count on the device, with and without
    maps: every filled row within the K/V bar, untouched slots unchanged, and
    within bf16 rounding of the int4 kernel's fill."""
    cfg = get_config(1, d=1024, n_tokens=640, n_slots=700)
    layers = [5, 6, 7]
    nl = len(layers)
    h = G.hidden_states(cfg, cfg.n_tokens, [4])[4].to(DEV)
    g = torch.Generator().manual_seed(77)
    slot = torch.randperm(cfg.n_slots, generator=g)[: cfg.n_tokens].to(torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    mp = G.near_identity_maps(cfg, nl).to(DEV) if maps else None
    sel = torch.sort(torch.randperm(cfg.n_tokens, generator=g)[:300]).values.to(torch.int32)
    rows = torch.full((cfg.n_tokens,), -1, dtype=torch.int32)
    rows[:300] = sel
    rows = rows.to(DEV)
    m_dev = torch.tensor([300], dtype=torch.int32, device=DEV)
    nh = cfg.n_kv_heads * cfg.head_dim
    # the automatic size holds the dequantised weights only where they would
    # be chosen; forcing them here needs their [nl][2 nh][d] bf16 on top
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, cfg.n_tokens, cfg.d, nh, 0, nl)
                     + nl * 2 * nh * cfg.d * 2, dtype=torch.uint8, device=DEV)
    out = {}
    try:
        for p in (2, 1):
            tee.river_debug_set_gemm_path(p)
            kc, vc = G.nan_cache(cfg, nl, device=DEV)
            tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=cfg.n_tokens,
                              m_dev=m_dev, row_idx=rows, maps=mp, workspace=ws)
            torch.cuda.synchronize()
            out[p] = (kc, vc)
    finally:
        tee.river_debug_set_gemm_path(0)
    kc, vc = out[2]
    check_fill(cfg, kc, vc, h, sel.numpy(), slot, mp, wk, wv)
    s_ = slot[sel.long().to(DEV)].long()
    for a, b in zip(out[2], out[1]):
        a, b = a[:, s_].float(), b[:, s_].float()
        assert torch.all((a - b).abs() <= 2 ** -6 * b.abs() + 1e-2 * b.abs().amax(dim=-1, keepdim=True))


@pytest.mark.parametrize("rows,nl,split", [(13, 3, False), (13, 3, True), (0, 3, True), (32, 17, True),
                                           (243, 1, True), (100, 12, True), (256, 2, False), (13, 21, True)])
def test_kv_fill_deep_projection(rows, nl, split):
    """Decode-sized projections (count on the device, bound 256, d = 4096,
    2 x 1024 outputs, group 128, bf16 scales) take the deep pipeline when its
    32-row tiles fit one round on the CUs, with a split over d chosen on the
    device when the workspace has room; more rows take the 128-row int4
    kernel (100 rows x 12 blocks: 384 tiles), in one launch that picks its
    side from the count when the 128-row side takes no split (21 or 12
    blocks here), else in two launches each idle for the other's counts.
    Without a split (no workspace, or 136 or 168 tiles at 32 rows) the caches
    equal the 128-row kernel's (gemm path 1) bit for bit; with one they agree
    to bf16 rounding. Every filled row is within the K/V bar, the other
    slots keep their sentinel; 0 rows write nothing."""
    cfg = get_config("3D")
    layers = list(range(5, 5 + nl))
    g = torch.Generator().manual_seed(4096 + rows)
    h = G.hidden_states(cfg, cfg.n_tokens, [4])[4].to(DEV)
    slot = torch.randperm(cfg.n_slots, generator=g)[: cfg.n_tokens].to(torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    sel = torch.sort(torch.randperm(cfg.n_tokens, generator=g)[:rows]).values.to(torch.int32)
    idx = torch.full((cfg.n_tokens,), -1, dtype=torch.int32)
    idx[:rows] = sel
    idx = idx.to(DEV)
    m_dev = torch.tensor([rows], dtype=torch.int32, device=DEV)
    nh = cfg.n_kv_heads * cfg.head_dim
    ws = None
    if split:
        ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, cfg.n_tokens, cfg.d, nh, 0, nl) + (16 << 20),
                         dtype=torch.uint8, device=DEV)
    out = {}
    try:
        for p in (0, 1):
            tee.river_debug_set_gemm_path(p)
            kc, vc = G.nan_cache(cfg, nl, device=DEV)
            tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=cfg.n_tokens,
                              m_dev=m_dev, row_idx=idx, workspace=ws if p == 0 else None)
            torch.cuda.synchronize()
            out[p] = (kc, vc)
    finally:
        tee.river_debug_set_gemm_path(0)
    kc, vc = out[0]
    if rows == 0:
        assert torch.isnan(kc.float()).all() and torch.isnan(vc.float()).all()
        return
    pick = np.linspace(0, rows - 1, min(rows, 24)).astype(np.int64)
    check_fill(cfg, kc, vc, h, sel.numpy(), slot, None, wk, wv, sample=pick)
    s_ = slot[sel.long().to(DEV)].long()
    bitwise = not split or (rows, nl) in ((32, 17), (100, 12), (13, 21))
    for a, b in zip(out[0], out[1]):
        if bitwise:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        else:
            a, b = a[:, s_].float(), b[:, s_].float()
            assert torch.all((a - b).abs() <= 2 ** -6 * b.abs() + 1e-3 * b.abs().amax(dim=-1, keepdim=True))


@pytest.mark.parametrize("d", [1280, 1024])
@pytest.mark.parametrize("count_on_device", [True, False])
def test_kv_fill_quad_tiles_equal_eight_wave_tiles(count_on_device, d):
    """The 256 x 256 tiles of the map GEMM and of the projection on
    dequantised weights run on the 4-wave kernels (gemm path 2: the ring of
    five 32 KB units at d = 1280, a multiple of 320; two 64 KB stages at d =
    1024) and on the 8-wave kernel (path 3). Both run the same MFMAs in the
    same order, so the caches agree bit for bit; the 4-wave result is within
    the K/V bar of the oracle. 300 of 640 rows (a ragged last tile), three
    layers, the count on the device or on the host."""
    cfg = get_config(1, d=d, n_tokens=640, n_slots=700)
    layers = [5, 6, 7]
    nl = len(layers)
    h = G.hidden_states(cfg, cfg.n_tokens, [4])[4].to(DEV)
    g = torch.Generator().manual_seed(160)
    slot = torch.randperm(cfg.n_slots, generator=g)[: cfg.n_tokens].to(torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, nl, scale=0.5).to(DEV)
    sel = torch.sort(torch.randperm(cfg.n_tokens, generator=g)[:300]).values.to(torch.int32)
    if count_on_device:
        rows = torch.full((cfg.n_tokens,), -1, dtype=torch.int32)
        rows[:300] = sel
        m_max, m_dev = cfg.n_tokens, torch.tensor([300], dtype=torch.int32, device=DEV)
    else:
        rows, m_max, m_dev = sel, 300, None
    rows = rows.to(DEV)
    nh = cfg.n_kv_heads * cfg.head_dim
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, m_max, cfg.d, nh, 0, nl)
                     + nl * 2 * nh * cfg.d * 2, dtype=torch.uint8, device=DEV)
    out = {}
    try:
        for p in (2, 3):
            tee.river_debug_set_gemm_path(p)
            kc, vc = G.nan_cache(cfg, nl, device=DEV)
            tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=m_max,
                              m_dev=m_dev, row_idx=rows, maps=maps, workspace=ws)
            torch.cuda.synchronize()
            out[p] = (kc, vc)
    finally:
        tee.river_debug_set_gemm_path(0)
    for a, b in zip(out[2], out[3]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    kc, vc = out[2]
    check_fill(cfg, kc, vc, h, sel.numpy(), slot, maps, wk, wv)


@pytest.mark.parametrize("d", [1280, 1152])
def test_kv_fill_quad_tiles_ragged_columns(d):
    """Column tiles that run past the output: 5 K/V heads of 64 (640
    projection columns, 2.5 tiles of 256) and, at d = 1152, 4.5 tiles of map
    columns (the two-stage 4-wave kernel; d = 1280 takes the ring). The
    4-wave kernels stage each tile's output in LDS and store only columns
    below N and rows below the count; they agree bit for bit with the 8-wave
    kernel and stay within the K/V bar of the oracle."""
    cfg = get_config(1, d=d, n_kv_heads=5, n_tokens=640, n_slots=700)
    layers = [5, 6]
    nl = len(layers)
    h = G.hidden_states(cfg, cfg.n_tokens, [4])[4].to(DEV)
    g = torch.Generator().manual_seed(161)
    slot = torch.randperm(cfg.n_slots, generator=g)[: cfg.n_tokens].to(torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, nl, scale=0.5).to(DEV)
    sel = torch.sort(torch.randperm(cfg.n_tokens, generator=g)[:333]).values.to(torch.int32)
    rows = sel.to(DEV)
    nh = cfg.n_kv_heads * cfg.head_dim
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, 333, cfg.d, nh, 0, nl)
                     + nl * 2 * nh * cfg.d * 2, dtype=torch.uint8, device=DEV)
    out = {}
    try:
        for p in (2, 3):
            tee.river_debug_set_gemm_path(p)
            kc, vc = G.nan_cache(cfg, nl, device=DEV)
            tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=333,
                              row_idx=rows, maps=maps, workspace=ws)
            torch.cuda.synchronize()
            out[p] = (kc, vc)
    finally:
        tee.river_debug_set_gemm_path(0)
    for a, b in zip(out[2], out[3]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    kc, vc = out[2]
    check_fill(cfg, kc, vc, h, sel.numpy(), slot, maps, wk, wv)


@pytest.mark.parametrize("d,heads,m,nl", [(768, 12, 3100, 3), (1280, 5, 1300, 2)])
def test_kv_fill_through_the_product_of_weights_and_maps(d, heads, m, nl):
    """From 4 n_out rows given on the host the plain fill with maps forms F =
    deq([Wk; Wv]) . maps per layer and projects the rows through it (the
    fill and the projection are both linear, so K and V are the same up to
    rounding). Both ways, through F and through x_hat (the fill-fuse hook),
    stay within the K/V bar of the oracle on every row, and agree with each
    other to it. d = 768 takes the two-stage 4-wave kernels; d = 1280 the
    ring, with 640 projection columns and F's 640 rows both ragged tiles of
    256. Ridge-fitted maps from the calibration states, rows in random
    order, slots a permutation."""
    cfg = get_config(1, d=d, n_kv_heads=heads, n_tokens=m + 200, n_slots=m + 300)
    e = 4
    layers = list(range(e + 1, e + 1 + nl))
    X, Y = G.calibration(cfg, e)
    maps = torch.from_numpy(O.ridge_fit(np64(X), np64(Y[:nl]), cfg.ridge_lambda)).to(torch.bfloat16).to(DEV)
    h = G.hidden_states(cfg, cfg.n_tokens, [e])[e].to(DEV)
    g = torch.Generator().manual_seed(162)
    slot = torch.randperm(cfg.n_slots, generator=g)[: cfg.n_tokens].to(torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    rows = torch.randperm(cfg.n_tokens, generator=g)[:m].to(torch.int32)
    nh = cfg.n_kv_heads * cfg.head_dim
    assert m >= 4 * nh
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, m, d, nh, 0, nl), dtype=torch.uint8, device=DEV)
    assert tee.river_debug_kv_fill_plan(m, d, nh, nl, ws.numel())[1] == 3
    out = {}
    try:
        for mode in (0, 1):
            tee.river_debug_set_fill_fuse(mode)
            kc, vc = G.nan_cache(cfg, nl, device=DEV)
            tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=m,
                              row_idx=rows.to(DEV), maps=maps, workspace=ws)
            torch.cuda.synchronize()
            out[mode] = (kc, vc)
    finally:
        tee.river_debug_set_fill_fuse(0)
    for mode in (0, 1):
        check_fill(cfg, *out[mode], h, rows.numpy(), slot, maps, wk, wv)
    s = slot[rows.to(DEV).long()].long()
    for a, b in zip(out[0], out[1]):
        x, y = a[:, s].float().reshape(nl, m, -1), b[:, s].float().reshape(nl, m, -1)
        err = (x - y).norm(dim=-1) / y.norm(dim=-1).clamp_min(1e-30)
        assert err.max().item() <= KV_TOL, err.max().item()


def test_kv_fill_times_its_gemm_launches_when_asked():
    """The measurement hook: with timing on, every chunk of a fill through
    the product leaves one timed product launch and one timed projection
    launch, each with a positive elapsed time; reading clears the records;
    with timing off the fill records nothing. The timed fill's K and V equal
    the untimed fill's bit for bit."""
    cfg = get_config(1, d=768, n_kv_heads=12, n_tokens=3300, n_slots=3400)
    m, nl, e = 3100, 3, 4
    layers = list(range(e + 1, e + 1 + nl))
    g = torch.Generator().manual_seed(163)
    maps = (torch.eye(cfg.d) + 0.02 * torch.randn(nl, cfg.d, cfg.d, generator=g)).to(torch.bfloat16).to(DEV)
    h = G.hidden_states(cfg, cfg.n_tokens, [e])[e].to(DEV)
    slot = torch.randperm(cfg.n_slots, generator=g)[: cfg.n_tokens].to(torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    rows = torch.randperm(cfg.n_tokens, generator=g)[:m].to(torch.int32).to(DEV)
    nh = cfg.n_kv_heads * cfg.head_dim
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, m, cfg.d, nh, 0, nl), dtype=torch.uint8,
                     device=DEV)
    chunk, path, _ = tee.river_debug_kv_fill_plan(m, cfg.d, nh, nl, ws.numel())
    assert path == 3
    chunks = -(-nl // chunk)
    for kind in (tee.TIMED_FILL_PROJECTION, tee.TIMED_FILL_PRODUCT):
        tee.river_debug_kernel_times(kind)
    out = []
    for on in (True, False):
        kc, vc = G.nan_cache(cfg, nl, device=DEV)
        tee.river_debug_time_kernels(on)
        try:
            tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=m, row_idx=rows,
                              maps=maps, workspace=ws)
        finally:
            tee.river_debug_time_kernels(False)
        torch.cuda.synchronize()
        out.append((kc, vc))
        for kind in (tee.TIMED_FILL_PROJECTION, tee.TIMED_FILL_PRODUCT):
            ms, n = tee.river_debug_kernel_times(kind)
            assert n == (chunks if on else 0), (on, kind, n)
            assert (ms > 0.0) if on else ms == 0.0, (on, kind, ms)
            assert tee.river_debug_kernel_times(kind) == (0.0, 0)
    for a, b in zip(out[0], out[1]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_kv_fill_identity_null_equals_explicit_eye():
    cfg = get_config(2)
    layers = list(range(9, 17))
    h = G.hidden_states(cfg, cfg.n_tokens, [8])[8].to(DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers)
    rows = torch.arange(0, 64, 2, dtype=torch.int32, device=DEV)
    k1, v1 = fill_gpu(cfg, h, slot, wk, wv, len(layers), row_idx=rows)
    eye = torch.eye(cfg.d, dtype=torch.bfloat16, device=DEV).expand(len(layers), -1, -1).contiguous()
    k2, v2 = fill_gpu(cfg, h, slot, wk, wv, len(layers), row_idx=rows, maps=eye)
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    check_fill(cfg, k1, v1, h, rows.cpu().numpy(), slot, None, wk, wv)


@pytest.mark.parametrize("n_layers,m", [(8, 37), (1, 64), (3, 1)])
def test_kv_fill_split_reduction_small_rows(n_layers, m):
    """At most 64 rows with room for partial sums: the reduction over d runs
    in parts whose fp32 sums a second kernel adds in a fixed order. Eight
    layers of the Llama-3.2-1B shape give 8 parts of 256 channels, one layer
    8 parts as well, three layers 2 parts. Within the K/V bar of the oracle,
    untouched slots unchanged, the same bits on a second call and the same
    rows as the unsplit projection to within bf16 rounding of the sum."""
    cfg = get_config(2)
    layers = list(range(cfg.L - n_layers + 1, cfg.L + 1))
    h = G.hidden_states(cfg, cfg.n_tokens, [cfg.L - n_layers])[cfg.L - n_layers].to(DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers)
    g = torch.Generator().manual_seed(m)
    sel = torch.randperm(cfg.n_tokens, generator=g)[:m].to(torch.int32)
    rows = torch.full((64,), -1, dtype=torch.int32)
    rows[:m] = sel
    rows = rows.to(DEV)
    m_dev = torch.tensor([m], dtype=torch.int32, device=DEV)
    nh = cfg.n_kv_heads * cfg.head_dim
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, 64, cfg.d, nh, 0, n_layers),
                     dtype=torch.uint8, device=DEV)
    out = []
    for w in (ws, ws, None):
        kc, vc = G.nan_cache(cfg, n_layers, device=DEV)
        tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=64,
                          m_dev=m_dev, row_idx=rows, workspace=w)
        torch.cuda.synchronize()
        out.append((kc, vc))
    (k1, v1), (k2, v2), (k0, v0) = out
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    check_fill(cfg, k1, v1, h, sel.numpy(), slot, None, wk, wv)
    s = slot[sel.long().to(DEV)].long()
    for a, b in ((k1, k0), (v1, v0)):
        a, b = a[:, s].float(), b[:, s].float()
        assert torch.all((a - b).abs() <= 2 ** -7 * b.abs() + 1e-4)


@pytest.mark.parametrize("m_small", [1, 20, 32])
def test_kv_fill_few_rows_on_device(m_small):
    """A count on the device of at most 32 rows under a bound of 200 (128-row
    tiles): the projection runs its loop on the first row fragment only.
    Within the K/V bar of the oracle, and bit for bit the rows that a count
    of 40 (the whole-tile loop) writes for the same first rows; other slots
    untouched."""
    cfg = get_config(1)
    n_layers, m_max, m_big = 3, 200, 40
    layers = list(range(cfg.L - n_layers + 1, cfg.L + 1))
    h = G.hidden_states(cfg, cfg.n_tokens, [cfg.L - n_layers])[cfg.L - n_layers].to(DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers)
    g = torch.Generator().manual_seed(7 + m_small)
    sel = torch.randperm(cfg.n_tokens, generator=g)[:m_big].to(torch.int32)
    rows = torch.full((m_max,), -1, dtype=torch.int32)
    rows[:m_big] = sel
    rows = rows.to(DEV)
    out = []
    for m in (m_small, m_big):
        kc, vc = G.nan_cache(cfg, n_layers, device=DEV)
        tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=m_max,
                          m_dev=torch.tensor([m], dtype=torch.int32, device=DEV), row_idx=rows)
        torch.cuda.synchronize()
        out.append((kc, vc))
    (k1, v1), (k2, v2) = out
    check_fill(cfg, k1, v1, h, sel[:m_small].numpy(), slot, None, wk, wv)
    s = slot[sel[:m_small].long().to(DEV)].long()
    assert torch.equal(k1[:, s].view(torch.int16), k2[:, s].view(torch.int16))
    assert torch.equal(v1[:, s].view(torch.int16), v2[:, s].view(torch.int16))


@pytest.mark.parametrize("n_layers,m,m_max", [(2, 150, 200), (1, 243, 256)])
def test_kv_fill_split_maps_and_projection(n_layers, m, m_max):
    """65 to 256 rows with few tiles and room for partial sums: the map GEMM
    and the projection both split the reduction over d (the map's parts are
    added before x-hat is rounded to bf16). Llama-3.2-1B shape with maps, the
    row count on the device and a ragged last row tile. Within the K/V bar
    of the oracle, the same bits on a second call, and the same rows as the
    unsplit fill (a workspace with room for the maps' outputs only) to
    within the bar."""
    cfg = get_config(2, n_tokens=m_max)
    layers = list(range(cfg.L - n_layers + 1, cfg.L + 1))
    h = G.hidden_states(cfg, cfg.n_tokens, [cfg.L - n_layers])[cfg.L - n_layers].to(DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, n_layers, tag=f"split{m}").to(DEV)
    g = torch.Generator().manual_seed(m)
    sel = torch.randperm(cfg.n_tokens, generator=g)[:m].to(torch.int32)
    rows = torch.full((m_max,), -1, dtype=torch.int32)
    rows[:m] = sel
    rows = rows.to(DEV)
    m_dev = torch.tensor([m], dtype=torch.int32, device=DEV)
    nh = cfg.n_kv_heads * cfg.head_dim
    big = tee.river_workspace_size(tee.OP_KV_FILL, m_max, cfg.d, nh, 0, n_layers)
    small = tee.river_workspace_size(tee.OP_KV_FILL, m_max, cfg.d, 0, 0, n_layers)
    assert big > small
    out = []
    for size in (big, big, small):
        ws = torch.empty(size, dtype=torch.uint8, device=DEV)
        kc, vc = G.nan_cache(cfg, n_layers, device=DEV)
        tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=m_max,
                          m_dev=m_dev, row_idx=rows, maps=maps, workspace=ws)
        torch.cuda.synchronize()
        out.append((kc, vc))
    (k1, v1), (k2, v2), (k0, v0) = out
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    check_fill(cfg, k1, v1, h, sel.numpy(), slot, maps, wk, wv)
    check_fill(cfg, k0, v0, h, sel.numpy(), slot, maps, wk, wv)
    s = slot[sel.long().to(DEV)].long()
    for a, b in ((k1, k0), (v1, v0)):
        a, b = a[:, s].float(), b[:, s].float()
        rel = (a - b).norm(dim=-1).norm(dim=-1) / b.norm(dim=-1).norm(dim=-1)
        assert float(rel.max()) <= 1e-2


@pytest.mark.parametrize("d,hkv,hd,group", [(200, 3, 24, 40), (512, 3, 24, 64), (264, 2, 32, 8)])
def test_kv_fill_bf16_generic_shapes(d, hkv, hd, group):
    """bf16 shapes the MFMA tiles do not take (d not a multiple of 256, an
    odd number of groups, n_out not a multiple of 64) run the generic
    kernel, with and without maps."""
    cfg = get_config(1, d=d, n_kv_heads=hkv, head_dim=hd, group=group, n_tokens=40, n_slots=96)
    layers = [5, 6, 7]
    h = G.hidden_states(cfg, cfg.n_tokens, [4])[4].to(DEV)
    g = torch.Generator().manual_seed(d)
    slot = torch.randperm(cfg.n_slots, generator=g)[: cfg.n_tokens].to(torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    rows = torch.tensor([1, 7, 39, 0, 22], dtype=torch.int32, device=DEV)
    maps = G.near_identity_maps(cfg, len(layers)).to(DEV)
    for mp in (None, maps):
        kc, vc = fill_gpu(cfg, h, slot, wk, wv, len(layers), row_idx=rows, maps=mp)
        check_fill(cfg, kc, vc, h, rows.cpu().numpy(), slot, mp, wk, wv)


def test_kv_fill_8b_sampled():
    cfg = get_config(3)
    e = 11
    layers = list(range(e + 1, cfg.L + 1))
    h = G.hidden_states(cfg, cfg.n_tokens, [e], device=DEV)[e]
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, len(layers), device=DEV)
    g = torch.Generator().manual_seed(11)
    sel = torch.sort(torch.randperm(cfg.n_tokens, generator=g)[:410]).values.to(torch.int32)
    kc, vc = fill_gpu(cfg, h, slot, wk, wv, len(layers), row_idx=sel.to(DEV), maps=maps)
    pick = np.sort(np.random.default_rng(1).choice(410, 24, replace=False))
    check_fill(cfg, kc, vc, h, sel.numpy(), slot, maps, wk, wv, sample=pick)


def test_kv_fill_long_context_sampled():
    cfg = get_config(4)
    e = 16
    n = cfg.n_tokens
    layers = list(range(e + 1, cfg.L + 1))
    h = G.hidden_states(cfg, n, [e], device=DEV)[e]
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers, device=DEV)
    maps = G.near_identity_maps(cfg, len(layers), device=DEV)
    rows = torch.arange(cfg.fill_lo, n - cfg.fill_tail, dtype=torch.int32, device=DEV)
    kc, vc = fill_gpu(cfg, h, slot, wk, wv, len(layers), row_idx=rows, maps=maps, ws_layers=6)
    m = rows.numel()
    pick = np.sort(np.random.default_rng(2).choice(m, 12, replace=False))
    pick[0] = 0
    pick[-1] = m - 1
    check_fill(cfg, kc, vc, h, rows.cpu().numpy(), slot, maps, wk, wv, sample=np.unique(pick))


# -------------------------------------------------------------- ridge fit

def ridge_gpu(X, Y, lam, wdt=torch.float32):
    T, n, d_out = Y.shape
    d_in = X.shape[1]
    W = torch.full((T, d_out, d_in), float("nan"), dtype=wdt, device=DEV)
    ws = torch.empty(tee.river_workspace_size(tee.OP_RIDGE_FIT, n, d_in, d_out, T,
                                              tee.RIVER_F32 if X.dtype == torch.float32 else tee.RIVER_BF16),
                     dtype=torch.uint8, device=DEV)
    tee.river_ridge_fit(X, Y, lam, W, workspace=ws)
    return W


def _rel_fro(a, b):
    return np.linalg.norm(np64(a) - b) / np.linalg.norm(b)


def test_ridge_fp32_tiny():
    cfg = get_config(0)
    X, Y = G.calibration(cfg, 2)
    ref = O.ridge_fit(np64(X), np64(Y), cfg.ridge_lambda)
    W = ridge_gpu(X.to(DEV), Y.to(DEV), cfg.ridge_lambda)
    assert _rel_fro(W, ref) <= 1e-3


@pytest.mark.parametrize("wdt,tol", [(torch.float32, 1e-3), (torch.bfloat16, 5e-3)])
def test_ridge_bf16_rectangular(wdt, tol):
    g = torch.Generator().manual_seed(21)
    n, d_in, d_out, T = 320, 128, 192, 3
    X = torch.randn(n, d_in, generator=g).bfloat16()
    Y = (torch.randn(T, n, d_out, generator=g) + X.float() @ torch.randn(d_in, d_out, generator=g) / 8).bfloat16()
    ref = O.ridge_fit(np64(X), np64(Y), 0.5)
    W = ridge_gpu(X.to(DEV), Y.to(DEV), 0.5, wdt)
    assert W.shape == (T, d_out, d_in)
    assert _rel_fro(W, ref) <= tol


def test_ridge_gpt2_maps():
    cfg = get_config(1)
    X, Y = G.calibration(cfg, 4)
    ref = O.ridge_fit(np64(X), np64(Y), cfg.ridge_lambda)
    W = ridge_gpu(X.to(DEV), Y.to(DEV), cfg.ridge_lambda, torch.bfloat16)
    assert _rel_fro(W, ref) <= 5e-3
    W32 = ridge_gpu(X.to(DEV), Y.to(DEV), cfg.ridge_lambda, torch.float32)
    assert _rel_fro(W32, ref) <= 1e-3
    # normal equations: (X^T X + lambda I) W^T = X^T Y
    Xd = np64(X)
    for t in (0, 7):
        Wt = np64(W32[t]).T
        res = Xd.T @ (Xd @ Wt) + cfg.ridge_lambda * Wt - Xd.T @ np64(Y[t])
        assert np.linalg.norm(res) <= 1e-4 * np.linalg.norm(Xd.T @ np64(Y[t]))


def test_ridge_not_spd():
    # a zero feature column with lambda = 0 gives an exactly zero pivot
    X = torch.randn(256, 128)
    X[:, 5] = 0
    X = X.bfloat16().to(DEV)
    Y = torch.randn(1, 256, 64).bfloat16().to(DEV)
    with pytest.raises(tee.RiverError) as e:
        ridge_gpu(X, Y, 0.0)
    assert e.value.name == "ERR_NOT_SPD"


def test_ridge_long_context_residual_sampled():
    cfg = get_config(4)
    X, Y = G.calibration(cfg, cfg.route_layers[0], device=DEV)
    Y = Y[:4].contiguous()
    W = ridge_gpu(X, Y, cfg.ridge_lambda)
    Xd = np64(X)
    rng = np.random.default_rng(3)
    for t in range(4):
        yt = np64(Y[t])
        for j in rng.choice(cfg.d, 4, replace=False):
            w = np64(W[t, j])
            res = Xd.T @ (Xd @ w) + cfg.ridge_lambda * w - Xd.T @ yt[:, j]
            assert np.linalg.norm(res) <= 1e-3 * np.linalg.norm(Xd.T @ yt[:, j])


# ------------------------------------------------------------ whole step

def test_step_gpt2_prefill_end_to_end():
    """route -> compact -> kv_fill, with the exit count passed on device."""
    cfg = get_config(1)
    e = 4
    layers = list(range(e + 1, cfg.L + 1))
    n = cfg.n_tokens
    hs = _states(cfg, n, [e - 1, e])
    wd, wu = (t.to(DEV) for t in G.router_weights(cfg, e))
    X, Y = G.calibration(cfg, e)
    maps = torch.from_numpy(O.ridge_fit(np64(X), np64(Y), cfg.ridge_lambda)).bfloat16().to(DEV)
    wk, wv = _kv(cfg, layers)
    slot = G.slots(cfg, device=DEV)
    mask = torch.empty(n, dtype=torch.uint8, device=DEV)
    cos = torch.empty(n, device=DEV)
    prob = torch.empty(n, device=DEV)
    tee.river_route(hs[e - 1], hs[e], mask, w_down=wd, w_up=wu, tau=cfg.tau, theta=cfg.theta,
                    cos_out=cos, prob_out=prob)
    cont = torch.empty(n, dtype=torch.int32, device=DEV)
    ext = torch.empty(n, dtype=torch.int32, device=DEV)
    counts = torch.empty(2, dtype=torch.int32, device=DEV)
    out = torch.full((n, cfg.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(tee.river_workspace_size(tee.OP_COMPACT, n), dtype=torch.uint8, device=DEV)
    tee.river_compact(mask, hs[e], cont, ext, counts, out=out, workspace=ws)
    kc, vc = fill_gpu(cfg, hs[e], slot, wk, wv, len(layers), row_idx=ext, m_dev=counts[1:],
                      m_max=n, maps=maps)
    ocos, oprob, omask, _ = route_ref(hs[e - 1], hs[e], wd, wu, cfg.tau, cfg.theta)
    band = (np.abs(ocos - f32(cfg.tau)) < BAND) | (np.abs(oprob - f32(cfg.theta)) < BAND)
    gm = mask.cpu().numpy()
    assert np.array_equal(gm[~band], omask[~band])
    # compaction of the GPU's own mask
    ref = O.compact(gm, None)
    ne = int(ref["counts"][1])
    assert counts.cpu().tolist() == [int(ref["counts"][0]), ne]
    assert np.array_equal(ext.cpu().numpy()[:ne], ref["exit_idx"])
    if not band.any():
        assert np.array_equal(ref["exit_idx"], np.flatnonzero(omask))
    ex = ref["exit_idx"]
    assert torch.equal(out[torch.from_numpy(ex).to(DEV)].view(torch.int16),
                       hs[e][torch.from_numpy(ex).to(DEV)].view(torch.int16))
    pick = np.sort(np.random.default_rng(4).choice(ne, 128, replace=False))
    check_fill(cfg, kc, vc, hs[e], ex, slot, maps, wk, wv, sample=pick)


def test_step_llama1b_decode_schedule():
    """River-LLM's token-level loop over layers 8..15 with the identity fill;
    per-layer tau splits the remaining tokens in half."""
    cfg = get_config(2)
    n = cfg.n_tokens
    hs = _states(cfg, n, range(7, 17))
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    kc, vc = G.nan_cache(cfg, cfg.L, device=DEV)
    alive = torch.arange(n, dtype=torch.int32, device=DEV)      # original rows still running
    exit_layer = np.full(n, cfg.L)
    for l in cfg.route_layers:
        hp, hc = hs[l - 1][alive.long()], hs[l][alive.long()]
        m = alive.numel()
        c, *_ = route_ref(hp, hc, None, None, -INF, -INF)
        srt = np.sort(c)
        tau = 0.5 * (srt[(m - 1) // 2] + srt[m // 2]) if m > 1 else srt[0] - 1
        mask = torch.empty(m, dtype=torch.uint8, device=DEV)
        alle = torch.empty(1, dtype=torch.int32, device=DEV)
        tee.river_route(hp, hc, mask, tau=tau, rule=O.RULE_TOKEN, all_exit_out=alle)
        cont = torch.empty(m, dtype=torch.int32, device=DEV)
        ext = torch.empty(m, dtype=torch.int32, device=DEV)
        counts = torch.empty(2, dtype=torch.int32, device=DEV)
        ridc = torch.empty(m, dtype=torch.int32, device=DEV)
        ws = torch.empty(tee.river_workspace_size(tee.OP_COMPACT, m), dtype=torch.uint8, device=DEV)
        tee.river_compact(mask, hc, cont, ext, counts, row_ids=alive, row_ids_cont=ridc, workspace=ws)
        nl = cfg.L - l
        sub = lambda w: tuple(t[l:] for t in w[:3]) + (w[3],)
        slot_alive = slot[alive.long()].contiguous()
        tee.river_kv_fill(hc, slot_alive, sub(wk), sub(wv), cfg.n_kv_heads, cfg.head_dim,
                          kc[l:], vc[l:], m_max=m, m_dev=counts[1:], row_idx=ext)
        torch.cuda.synchronize()
        gm = mask.cpu().numpy()
        _, _, om, _ = route_ref(hp, hc, None, None, tau, -INF)
        band = np.abs(c - f32(tau)) < BAND
        assert np.array_equal(gm[~band], om[~band])
        assert int(alle.item()) == int(gm.all())
        nc, ne = counts.cpu().tolist()
        a = alive.cpu().numpy()
        exit_layer[a[gm != 0]] = l
        alive = ridc[:nc].clone()
        assert np.array_equal(alive.cpu().numpy(), a[gm == 0])
        if nc == 0:
            break
    # every token that exited at l has layers l+1..16 filled and nothing else
    hs_np = {l: np64(hs[l]) for l in range(7, 17)}
    for t in range(n):
        e = exit_layer[t]
        s = int(slot[t])
        filled = ~torch.isnan(kc[:, s]).all(dim=-1).all(dim=-1).cpu().numpy()
        assert np.array_equal(filled, np.arange(1, cfg.L + 1) > e)
        if e < cfg.L:
            K, V = O.kv_fill_rows(hs_np[e][t:t + 1], None, 1, None,
                                  {k: (v[e:] if k != "group" else v) for k, v in w4_np(wk).items()},
                                  {k: (v[e:] if k != "group" else v) for k, v in w4_np(wv).items()})
            assert kv_row_errors(kc[e:, s].reshape(cfg.L - e, 1, -1), K).max() <= KV_TOL
            assert kv_row_errors(vc[e:, s].reshape(cfg.L - e, 1, -1), V).max() <= KV_TOL
    assert (exit_layer < cfg.L).sum() >= n // 2
