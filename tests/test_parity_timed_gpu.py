"""GPU parity at the shapes, and on the paths, that the benchmark times.

Each test builds the benchmark's own workload object (bench.py: the same
calls, the same workspace sizes and so the same launch paths), runs one
step on NaN-filled caches and checks it against the float64 oracle:

* the long-context prefill at 32,768 and 65,536 tokens (d = 5120, 48
  filled layers, through the product of the dequantised weights and the
  maps);
* the Llama-3-8B prefill step over all eight checkpoints (route, compaction
  with the gather and the exit scatter, the fills at blocks 11 and 31);
* the GPT-2-shape step (route, compaction with the gather and the exit
  scatter, the fill with the count on the device);
* river_ridge_fit at the long-context and 8B calibration sizes.

The fills take ridge maps fitted by the oracle (float64, from the same
calibration states the benchmark fits its maps from, rounded to bf16): an
input of the oracle never comes from the library. Where a fill has more
layers than the oracle fits maps for in seconds, the fitted maps repeat
over the layers in turn, so that neighbouring layers differ.

Bars: masks, indices and counts bit-exact (tokens within 1e-4 of a
threshold excluded and counted); copied rows bitwise equal; K/V per-row
relative L2 <= 1e-2 on sampled rows (the first and last row of every
256-row tile of the fill and random others, at least 1024 where the fill
has that many) over every filled layer; every slot not filled keeps its
NaN sentinel and every filled one holds no NaN; ridge maps within 5e-3
relative Frobenius (bf16 output) on sampled output rows of every target.
"""

import math

import numpy as np
import pytest
import torch

import bench as B
import oracle as O
import token_early_exit_amd as tee
from synth import get_config
from synth import generate as G
from helpers import BAND, KV_TOL, f32, kv_row_errors, midpoint_threshold, np64, w4_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
INF = math.inf


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    tee.river_debug_set_compact_path(0)
    tee.river_debug_set_gemm_path(0)
    yield


def tile_sample(m, k, seed, tile=256):
    """Positions of 0..m-1 to check: the first and last of every tile of the
    fill's rows, and random others up to k in all (or every position)."""
    if m <= k:
        return np.arange(m)
    first = np.arange(0, m, tile)
    base = np.union1d(first, np.minimum(first + tile - 1, m - 1))
    rest = np.setdiff1d(np.arange(m), base)
    extra = np.random.default_rng(seed).choice(rest, max(0, k - len(base)), replace=False)
    return np.sort(np.concatenate([base, extra]))


class Cycle:
    """Layer l takes base[l % len(base)]."""

    def __init__(self, base, n):
        self.base, self.n = base, n

    def __getitem__(self, l):
        if not 0 <= l < self.n:
            raise IndexError(l)
        return self.base[l % len(self.base)]


def oracle_maps(X, Y, targets, lam):
    """Ridge maps of the given targets fitted by the oracle, as bf16 (the
    dtype the fill takes) and as float32 copies of those bf16 values."""
    ref = O.ridge_fit(np64(X), np64(Y[list(targets)]), lam)
    mb = torch.from_numpy(ref).to(torch.bfloat16)
    return mb, mb.float().numpy()


def check_fill_rows(kc, vc, h_rows, slots, maps_np, wk, wv, n_layers):
    """Sampled rows' K/V in every filled cache layer against the oracle.
    kc, vc: the cache layers the fill wrote; h_rows: the rows' states;
    slots: their cache slots."""
    K, V = O.kv_fill_rows(h_rows, None, h_rows.shape[0], maps_np, w4_np(wk), w4_np(wv))
    s = torch.from_numpy(np.asarray(slots, dtype=np.int64)).to(DEV)
    gk = kc[:, s].reshape(n_layers, len(slots), -1)
    gv = vc[:, s].reshape(n_layers, len(slots), -1)
    ek, ev = kv_row_errors(gk, K), kv_row_errors(gv, V)
    assert ek.max() <= KV_TOL and ev.max() <= KV_TOL, (ek.max(), ev.max())
    return max(ek.max(), ev.max())


def check_sentinel(kc, vc, filled):
    """Per cache layer: the filled slots hold no NaN, every other slot is
    all NaN. filled: bool [layers][n_slots] on the device."""
    for l in range(kc.shape[0]):
        for c in (kc, vc):
            anynan = torch.isnan(c[l]).flatten(1).any(dim=1)
            allnan = torch.isnan(c[l]).flatten(1).all(dim=1)
            f = filled[l]
            assert not bool(anynan[f].any()), f"layer {l}: a filled slot holds NaN"
            assert bool(allnan[~f].all()), f"layer {l}: a slot that was not filled changed"


# ------------------------------------------------------- long context

@pytest.fixture(scope="module")
def long_calibration():
    """The long-context calibration pair (16,384 tokens, 48 targets) on the
    device, the oracle's ridge maps of three targets (first, middle, last)
    and the sampled output columns of every target."""
    cfg = get_config(4)
    X, Y = G.calibration(cfg, cfg.route_layers[0], device=DEV)
    mb, mf = oracle_maps(X, Y, (0, 23, 47), cfg.ridge_lambda)
    yield cfg, X, Y, mb, mf


def test_ridge_fit_long_context_full(long_calibration):
    """river_ridge_fit as the benchmark calls it: 48 maps of 5120 x 5120 from
    16,384 calibration tokens, lambda = 0.1, bf16 output; twelve output rows
    of every target against the oracle's solve of the same columns (ridge is
    column by column, so one solve with those columns of every target
    stacked gives exactly those rows of every map)."""
    cfg, X, Y, _, _ = long_calibration
    T, n, d = Y.shape
    W = torch.full((T, d, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(tee.river_workspace_size(tee.OP_RIDGE_FIT, n, d, d, T, tee.RIVER_BF16),
                     dtype=torch.uint8, device=DEV)
    tee.river_ridge_fit(X, Y, cfg.ridge_lambda, W, workspace=ws)
    cols = np.unique(np.concatenate([[0, d - 1], np.random.default_rng(4).choice(d, 10, replace=False)]))
    ci = torch.from_numpy(cols).to(DEV)
    Ys = Y[:, :, ci].permute(1, 0, 2).reshape(1, n, T * len(cols))     # [1][n][T * cols]
    ref = O.ridge_fit(np64(X), np64(Ys), cfg.ridge_lambda)[0].reshape(T, len(cols), d)
    got = np64(W[:, ci, :])
    assert not np.isnan(got).any()
    for t in range(T):
        rel = np.linalg.norm(got[t] - ref[t]) / np.linalg.norm(ref[t])
        assert rel <= 5e-3, (t, rel)


@pytest.mark.parametrize("N,folded", [(32768, False), (65536, False), (65536, True)])
def test_long_context_step(long_calibration, N, folded):
    """One step of the benchmark's long-context workload: the positional
    compaction, then the fill of every row between the first 16 and the
    last 2048 through 48 layers on the path the benchmark times (per layer
    the product F = deq([Wk; Wv]) . maps, then the rows through F); folded:
    the step with F formed once beforehand (river_kv_fold, then
    river_kv_fill_folded)."""
    cfg0, _, _, mb, mf = long_calibration
    nl = 48
    wl = B.LongContextWorkload(N, maps=Cycle(mb, nl))
    cfg = wl.cfg
    m, d = wl.m, cfg.d
    assert m == N - cfg.fill_lo - cfg.fill_tail
    assert tee.river_debug_kv_fill_plan(m, d, wl.n_out, nl, wl.ws.numel()) == (nl, 3, 1)
    wl.kc.fill_(float("nan"))
    wl.vc.fill_(float("nan"))
    if folded:
        wl.fold()
        wl.step_folded()
    else:
        wl.step()
    torch.cuda.synchronize()
    # compaction of the positional mask: bit-exact
    assert wl.counts.cpu().tolist() == [N - m, m]
    assert np.array_equal(wl.ext[:m].cpu().numpy(), np.arange(cfg.fill_lo, N - cfg.fill_tail))
    assert np.array_equal(wl.cont[:N - m].cpu().numpy(),
                          np.concatenate([np.arange(cfg.fill_lo), np.arange(N - cfg.fill_tail, N)]))
    # K/V of sampled rows over all 48 layers
    pick = tile_sample(m, 1024, N)
    rows = cfg.fill_lo + pick
    h_rows = wl.h[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    slots = wl.slot.cpu().numpy()[rows]
    check_fill_rows(wl.kc, wl.vc, h_rows, slots, Cycle(mf, nl), wl.wk, wl.wv, nl)
    # exactly the rows 16..N-2048 of every layer were written
    filled = torch.zeros(N, dtype=torch.bool, device=DEV)
    filled[cfg.fill_lo:N - cfg.fill_tail] = True
    check_sentinel(wl.kc, wl.vc, filled.expand(nl, N))


# ------------------------------------------------------- 8B prefill step

@pytest.fixture(scope="module")
def prefill_8b_inputs():
    """Oracle thresholds and ridge maps of the 8B prefill: theta at block 11
    between the oracle's 410th and 411th largest probabilities; maps for the
    exits at 11 (targets 0, 10, 20 of blocks 12..32, repeating over the 21
    layers) and at 31 (block 32), fitted by the oracle from the 8192
    calibration tokens."""
    cfg = get_config(3)
    n = cfg.n_tokens
    e1, e2 = cfg.extra["exit_early"], cfg.extra["exit_late"]
    hs = G.hidden_states(cfg, n, [e1 - 1, e1], device=DEV)
    wd, wu = G.router_weights(cfg, e1, device=DEV)
    _, prob, _, _ = O.route(np64(hs[e1 - 1]), np64(hs[e1]), None, 1e-6, np64(wd), np64(wu), -INF, -INF)
    theta11 = midpoint_threshold(prob, int(round(cfg.extra["early_frac"] * n)))
    X, Y = G.calibration(cfg, e1, device=DEV)
    mb1, mf1 = oracle_maps(X, Y, (0, 10, 20), cfg.ridge_lambda)
    del X, Y
    X, Y = G.calibration(cfg, e2, device=DEV)
    mb2, mf2 = oracle_maps(X, Y, (0,), cfg.ridge_lambda)
    del X, Y, hs
    torch.cuda.empty_cache()
    return cfg, theta11, (mb1, mf1), (mb2, mf2)


@pytest.mark.parametrize("folded", [False, True])
def test_prefill_8b_step(prefill_8b_inputs, folded):
    """One step of the benchmark's 8B prefill workload: every checkpoint's
    decision against the oracle's (outside the band), the compaction of the
    GPU's own masks (indices, counts, gathered rows and ids, exit scatter)
    bit-exact, the fills at 11 (every exited row, 21 layers) and 31 (sampled
    rows of 7782, one layer) within the K/V bar, and every other cache slot
    untouched; folded: the fills through river_kv_fold's products."""
    cfg, theta11, (mb1, mf1), (mb2, mf2) = prefill_8b_inputs
    wl = B.Prefill8BWorkload(theta11=theta11, maps11=torch.stack([Cycle(mb1, 21)[l] for l in range(21)]),
                             maps31=mb2)
    n, L = wl.n, cfg.L
    assert wl.theta[wl.e1] == theta11
    if folded:
        wl.fold()               # the fills through deq([Wk; Wv]) M, as the benchmark's folded step
    wl.kc.fill_(float("nan"))
    wl.vc.fill_(float("nan"))
    wl.out.fill_(float("nan"))
    wl.step()
    torch.cuda.synchronize()
    exit_layer = np.full(n, L)
    for c in wl.CKS:
        s = wl.ck[c]
        hp, hc = np64(s["hp"]), np64(s["hc"])
        wd, wu = (np64(t) for t in wl.routers[c])
        _, prob, om, _ = O.route(hp, hc, None, 1e-6, wd, wu, -INF, f32(wl.theta[c]))
        gm = s["mask"].cpu().numpy()
        band = np.abs(prob - f32(wl.theta[c])) < BAND
        assert band.sum() <= 2, (c, band.sum())
        assert np.array_equal(gm[~band], om[~band]), c
        ids = np.arange(s["n"]) if s["ids"] is None else s["ids"].cpu().numpy()
        ref = O.compact(gm, hc, ids, None)
        nc, ne = (int(x) for x in ref["counts"])
        assert s["counts"].cpu().tolist() == [nc, ne]
        assert np.array_equal(s["cont"][:nc].cpu().numpy(), ref["cont_idx"])
        assert np.array_equal(s["ext"][:ne].cpu().numpy(), ref["exit_idx"])
        assert np.array_equal(s["ids_cont"][:nc].cpu().numpy(), ref["row_ids_cont"])
        if nc:
            ci = torch.from_numpy(ref["cont_idx"]).to(DEV)
            assert torch.equal(s["h_cont"][:nc].view(torch.int16), s["hc"][ci].view(torch.int16))
        if ne:
            ei = torch.from_numpy(ref["exit_idx"]).to(DEV)
            dst = torch.from_numpy(ids[ref["exit_idx"]]).to(DEV)
            assert torch.equal(wl.out[dst].view(torch.int16), s["hc"][ei].view(torch.int16))
            exit_layer[ids[ref["exit_idx"]]] = c
    assert wl.exits[wl.e1] == int((exit_layer == wl.e1).sum())
    assert abs(wl.exits[wl.e1] - 410) <= 2 and (exit_layer == wl.e2).sum() == n - wl.exits[wl.e1]
    # every token's final state is in out
    assert not bool(torch.isnan(wl.out).any())
    # fills: at 11 every exited row over blocks 12..32, at 31 sampled rows
    s1 = wl.ck[wl.e1]
    ex1 = s1["ext"][:wl.exits[wl.e1]].cpu().numpy()
    check_fill_rows(wl.kc[L - 21:], wl.vc[L - 21:], np64(s1["hc"])[ex1], ex1, Cycle(mf1, 21), wl.wk1, wl.wv1, 21)
    s2 = wl.ck[wl.e2]
    m2 = wl.exits[wl.e2]
    pick = tile_sample(m2, 1024, 31)
    ex2 = s2["ext"][:m2].cpu().numpy()[pick]
    slots2 = s2["ids"].cpu().numpy()[ex2]
    check_fill_rows(wl.kc[L - 1:], wl.vc[L - 1:], np64(s2["hc"][torch.from_numpy(ex2).to(DEV)]), slots2,
                    mf2, wl.wk2, wl.wv2, 1)
    # cache layer j-1 holds block j: filled exactly for tokens with exit layer < j
    el = torch.from_numpy(exit_layer).to(DEV)
    blocks = torch.arange(1, L + 1, device=DEV)[:, None]
    check_sentinel(wl.kc, wl.vc, blocks > el[None, :])


def test_ridge_fit_8b_prefill_sampled():
    """river_ridge_fit as the 8B prefill workload calls it: the 21 maps of
    exit 11 from 8192 calibration tokens (lambda = 0.1, bf16 output); ten
    output rows of every target against the oracle."""
    cfg = get_config(3)
    X, Y = G.calibration(cfg, cfg.extra["exit_early"], device=DEV)
    T, n, d = Y.shape
    W = torch.full((T, d, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(tee.river_workspace_size(tee.OP_RIDGE_FIT, n, d, d, T, tee.RIVER_BF16),
                     dtype=torch.uint8, device=DEV)
    tee.river_ridge_fit(X, Y, cfg.ridge_lambda, W, workspace=ws)
    cols = np.unique(np.concatenate([[0, d - 1], np.random.default_rng(8).choice(d, 8, replace=False)]))
    ci = torch.from_numpy(cols).to(DEV)
    Ys = Y[:, :, ci].permute(1, 0, 2).reshape(1, n, T * len(cols))
    ref = O.ridge_fit(np64(X), np64(Ys), cfg.ridge_lambda)[0].reshape(T, len(cols), d)
    got = np64(W[:, ci, :])
    for t in range(T):
        rel = np.linalg.norm(got[t] - ref[t]) / np.linalg.norm(ref[t])
        assert rel <= 5e-3, (t, rel)


# ------------------------------------------------------- GPT-2-shape step

def test_gpt2_step():
    """One step of the benchmark's GPT-2-shape workload (oracle ridge maps):
    the route against the oracle outside the band, the compaction of the
    GPU's mask with the gather and the exit scatter bit-exact, the fill of
    the exited rows (count on the device) within the K/V bar."""
    cfg = get_config(1)
    e = cfg.route_layers[0]
    X, Y = G.calibration(cfg, e)
    maps = torch.from_numpy(O.ridge_fit(np64(X), np64(Y), cfg.ridge_lambda)).to(torch.bfloat16)
    wl = B.Gpt2Workload(1, maps=maps)
    s = wl.sets[0]
    s["kc"].fill_(float("nan"))
    s["vc"].fill_(float("nan"))
    s["out"].fill_(float("nan"))
    wl.step(0)
    torch.cuda.synchronize()
    hc = np64(wl.h_cur0)
    ocos, oprob, om, _ = O.route(np64(wl.h_prev0), hc, None, 1e-6, np64(wl.wd), np64(wl.wu),
                                 f32(cfg.tau), f32(cfg.theta))
    gm = s["mask"].cpu().numpy()
    band = (np.abs(ocos - f32(cfg.tau)) < BAND) | (np.abs(oprob - f32(cfg.theta)) < BAND)
    assert np.array_equal(gm[~band], om[~band])
    ref = O.compact(gm, hc, None, None)
    nc, ne = (int(x) for x in ref["counts"])
    assert s["counts"].cpu().tolist() == [nc, ne]
    assert np.array_equal(s["ext"][:ne].cpu().numpy(), ref["exit_idx"])
    assert np.array_equal(s["cont"][:nc].cpu().numpy(), ref["cont_idx"])
    ci = torch.from_numpy(ref["cont_idx"]).to(DEV)
    ei = torch.from_numpy(ref["exit_idx"]).to(DEV)
    assert torch.equal(s["h_cont"][:nc].view(torch.int16), s["hc"][ci].view(torch.int16))
    assert torch.equal(s["out"][ei].view(torch.int16), s["hc"][ei].view(torch.int16))
    assert bool(torch.isnan(s["out"][ci]).all())
    pick = tile_sample(ne, 1024, 1)
    ex = ref["exit_idx"][pick]
    check_fill_rows(s["kc"], s["vc"], hc[ex], wl.slot.cpu().numpy()[ex], maps.float().numpy(), wl.wk, wl.wv,
                    wl.nl)
    filled = torch.zeros(cfg.n_slots, dtype=torch.bool, device=DEV)
    filled[wl.slot[ei].long()] = True
    check_sentinel(s["kc"], s["vc"], filled.expand(wl.nl, -1))
