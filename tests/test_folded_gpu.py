"""GPU parity of the folded fill.

RidgeFill 思路源头: a skipped layer's K/V come from its own projection of
the input a fitted map predicts. river_kv_fold composes the two per layer,
F = deq([Wk; Wv]) . M, and river_kv_fill_folded (or a decode checkpoint
with folded products) projects the exit states through F. Checked here
against the float64 oracle's two-step fill (x_hat = M x, then the int4
projection) on the same maps and int4 weights, and F itself against the
product of the oracle's dequantised weights and the maps.

Bars: F per-row relative L2 <= 1e-2 (one bf16 rounding of each element);
K/V per-row relative L2 <= 1e-2; every slot not filled keeps its NaN
sentinel. The maps are I + N(0, 1/d) (as large a random part as the
identity), so that a transposed or misplaced map shows.
"""

import numpy as np
import pytest
import torch

import bench as B
import oracle as O
import token_early_exit_amd as tee
from synth import get_config
from synth import generate as G
from helpers import KV_TOL, kv_row_errors, np64, w4_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    tee.river_debug_set_gemm_path(0)
    yield


def weights(cfg, nl):
    w = G.kv_weights(cfg, list(range(1, nl + 1)), device=DEV)
    return B.kv_tuple(w, "wk", cfg.group), B.kv_tuple(w, "wv", cfg.group)


@pytest.mark.parametrize("key,nl,with_maps", [(1, 3, True), (2, 2, True), (2, 2, False)])
def test_kv_fold_against_the_oracle_product(key, nl, with_maps):
    cfg = get_config(key)
    d, n_out = cfg.d, cfg.n_kv_heads * cfg.head_dim
    wk, wv = weights(cfg, nl)
    maps = G.near_identity_maps(cfg, nl, scale=1.0, tag="fold", device=DEV) if with_maps else None
    F = torch.full((nl, 2 * n_out, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = None
    if with_maps:
        # a workspace for one layer: the layers go in passes of one
        ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FOLD, 0, d, n_out, 0, 1), dtype=torch.uint8,
                         device=DEV)
    tee.river_kv_fold(wk, wv, cfg.n_kv_heads, cfg.head_dim, F, maps=maps, workspace=ws)
    torch.cuda.synchronize()
    Wk = O.dequant_w4(*[w4_np(wk)[k] for k in ("q", "scale", "zero", "group")])
    Wv = O.dequant_w4(*[w4_np(wv)[k] for k in ("q", "scale", "zero", "group")])
    W = np.concatenate([Wk, Wv], axis=1)                          # [nl][2 n_out][d]
    ref = W if maps is None else W @ np64(maps)
    err = kv_row_errors(F, ref)
    assert err.max() <= KV_TOL, err.max()


def run_folded(cfg, nl, n_rows, m_max, m_dev, row_idx, maps, wk, wv):
    d, n_out = cfg.d, cfg.n_kv_heads * cfg.head_dim
    h = G.hidden_states(cfg, n_rows, [1], tag="folded", device=DEV)[1]
    slot = torch.randperm(cfg.n_slots, generator=torch.Generator().manual_seed(5))[:n_rows].to(torch.int32).to(DEV)
    F = torch.empty((nl, 2 * n_out, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FOLD, 0, d, n_out, 0, nl), dtype=torch.uint8, device=DEV)
    tee.river_kv_fold(wk, wv, cfg.n_kv_heads, cfg.head_dim, F, maps=maps, workspace=ws)
    kc, vc = G.nan_cache(cfg, nl, device=DEV)
    tee.river_kv_fill_folded(h, slot, F, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=m_max, m_dev=m_dev,
                             row_idx=row_idx)
    torch.cuda.synchronize()
    return h, slot, kc, vc


@pytest.mark.parametrize("case", ["host-700-of-1000", "device-37-of-200", "device-410-of-2048", "empty"])
def test_kv_fill_folded_against_the_oracle(case):
    """Host count on the 256 x 256 tiles with a ragged last tile (700 rows
    picked from 1000, d = 768); device counts on the 32-row tiles (37 of a
    bound of 200, d = 2048) and on the 256 x 256 tiles (410 of 2048); a
    device count of 0."""
    key, n_rows, m_max, m = {"host-700-of-1000": (1, 1000, 700, 700),
                             "device-37-of-200": (2, 300, 200, 37),
                             "device-410-of-2048": (2, 2048, 2048, 410),
                             "empty": (2, 300, 200, 0)}[case]
    cfg = get_config(key)
    nl = 3
    wk, wv = weights(cfg, nl)
    maps = G.near_identity_maps(cfg, nl, scale=1.0, tag="fill", device=DEV)
    rows = np.sort(np.random.default_rng(3).choice(n_rows, m_max, replace=False)).astype(np.int32)
    row_idx = torch.from_numpy(rows).to(DEV)
    m_dev = None if case.startswith("host") else torch.tensor([m], dtype=torch.int32, device=DEV)
    h, slot, kc, vc = run_folded(cfg, nl, n_rows, m_max, m_dev, row_idx, maps, wk, wv)
    filled = rows[:m]
    slot_np = slot.cpu().numpy()
    if m:
        pick = filled if m <= 256 else np.sort(np.random.default_rng(4).choice(filled, 256, replace=False))
        K, V = O.kv_fill_rows(np64(h), pick, len(pick), maps.float().cpu().numpy(), w4_np(wk), w4_np(wv))
        s = torch.from_numpy(slot_np[pick].astype(np.int64)).to(DEV)
        ek = kv_row_errors(kc[:, s].reshape(nl, len(pick), -1), K)
        ev = kv_row_errors(vc[:, s].reshape(nl, len(pick), -1), V)
        assert ek.max() <= KV_TOL and ev.max() <= KV_TOL, (ek.max(), ev.max())
    want = np.zeros(cfg.n_slots, bool)
    want[slot_np[filled]] = True
    for c in (kc, vc):
        isnan = torch.isnan(c).flatten(2).all(dim=2).cpu().numpy()      # [nl][n_slots]
        anynan = torch.isnan(c).flatten(2).any(dim=2).cpu().numpy()
        assert np.array_equal(isnan, np.broadcast_to(~want, isnan.shape))
        assert not anynan[:, want].any()
