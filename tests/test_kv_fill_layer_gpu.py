"""GPU parity of the fill through the skipped layers' full K/V path
(river_kv_fill_layer: input RMSNorm, K/V bias, rotary embedding of K)
against the float64 oracle.

Bar: per-row relative L2 error of every filled K and V row <= 1e-2 (the
fill's bar: the GPU rounds the layer input to bf16 before the int4
projection, the oracle keeps float64); slots that receive nothing keep
their NaN sentinel; with no layer part switched on the result equals
river_kv_fill bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle as O
import token_early_exit_amd as tee
from synth import get_config
from synth import generate as G
from helpers import KV_TOL, kv_row_errors, np64, w4_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


def _kv(cfg, layers):
    w = G.kv_weights(cfg, layers, device="cpu" if cfg.d <= 2048 else DEV)
    wk = tuple(t.to(DEV) for t in w["wk"]) + (cfg.group,)
    wv = tuple(t.to(DEV) for t in w["wv"]) + (cfg.group,)
    return wk, wv


def _parts(cfg, layers, norm=True, bias=True, rope=True, n_pos=None):
    p = {}
    if norm:
        p["norm_gamma"] = G.layer_norm_gammas(cfg, layers).to(DEV)
        p["norm_eps"] = 1e-5
    if bias:
        bk, bv = G.kv_biases(cfg, layers)
        p["k_bias"], p["v_bias"] = bk.to(DEV), bv.to(DEV)
    if rope:
        c, s = G.rope_tables(cfg, n_pos or cfg.n_slots)
        p["rope_cos"], p["rope_sin"] = c.to(DEV), s.to(DEV)
    return p


def fill_layer_gpu(cfg, h, slot, wk, wv, n_layers, parts, pos=None, row_idx=None, m_dev=None,
                   m_max=None, maps=None, ws_layers=None):
    shape = (n_layers, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim)
    dt = h.dtype
    kc = torch.full(shape, float("nan"), dtype=dt, device=DEV)
    vc = torch.full(shape, float("nan"), dtype=dt, device=DEV)
    mm = m_max if m_max is not None else (row_idx.shape[0] if row_idx is not None else h.shape[0])
    ws = None
    if maps is not None or "norm_gamma" in parts:
        nl = n_layers if ws_layers is None else ws_layers
        ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL_LAYER, mm, cfg.d, 0, 0, nl),
                         dtype=torch.uint8, device=DEV)
    tee.river_kv_fill_layer(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=mm,
                            m_dev=m_dev, row_idx=row_idx, maps=maps, pos=pos if "rope_cos" in parts else None,
                            workspace=ws, **parts)
    torch.cuda.synchronize()
    return kc, vc


def check_layer(cfg, kc, vc, h, rows, slot, maps, wk, wv, parts, pos, sample=None, skipped=()):
    rows = np.asarray(rows)
    slot_np = slot.cpu().numpy()
    pick = np.arange(len(rows)) if sample is None else np.asarray(sample)
    pick = np.array([i for i in pick if rows[i] not in set(skipped)], dtype=np.int64)
    g = lambda k: None if k not in parts else np64(parts[k])
    rope = "rope_cos" in parts
    K, V = O.kv_fill_layer_rows(np64(h), rows[pick], len(pick),
                                None if maps is None else maps.float().cpu().numpy(),
                                w4_np(wk), w4_np(wv), g("norm_gamma"),
                                float(np.float32(parts.get("norm_eps", 0.0))), g("k_bias"),
                                g("v_bias"), pos.cpu().numpy() if rope else None, g("rope_cos"),
                                g("rope_sin"), cfg.n_kv_heads, cfg.head_dim)
    s = torch.from_numpy(slot_np[rows[pick]].astype(np.int64)).to(DEV)
    ek = kv_row_errors(kc[:, s].reshape(kc.shape[0], len(pick), -1), K)
    ev = kv_row_errors(vc[:, s].reshape(vc.shape[0], len(pick), -1), V)
    assert ek.max() <= KV_TOL and ev.max() <= KV_TOL, (ek.max(), ev.max())
    filled = torch.zeros(kc.shape[1], dtype=torch.bool)
    done = [r for r in rows if r not in set(skipped)]
    filled[torch.from_numpy(slot_np[done].astype(np.int64))] = True
    nan_k = torch.isnan(kc).all(dim=-1).all(dim=-1).cpu()
    nan_v = torch.isnan(vc).all(dim=-1).all(dim=-1).cpu()
    assert torch.all(nan_k[:, ~filled]) and not torch.any(nan_k[:, filled])
    assert torch.all(nan_v[:, ~filled]) and not torch.any(nan_v[:, filled])
    return ek.max(), ev.max()


def test_layer_fill_llama1b_decode_identity():
    """Llama-3.2-1B-shape decode: 64 tokens at distinct slots, the identity
    map, the layer's input RMSNorm and RoPE at the token positions."""
    cfg = get_config(2)
    layers = list(range(9, 17))
    h = G.hidden_states(cfg, cfg.n_tokens, [8])[8].to(DEV)
    slot = G.slots(cfg, device=DEV)
    pos = slot.clone()                         # a decode token's position is its slot
    wk, wv = _kv(cfg, layers)
    parts = _parts(cfg, layers, bias=False)
    sel = torch.arange(0, 64, 3, dtype=torch.int32)
    rows = torch.full((64,), -1, dtype=torch.int32)        # row_idx holds m_max entries
    rows[: sel.numel()] = sel
    m_dev = torch.tensor([sel.numel()], dtype=torch.int32, device=DEV)
    kc, vc = fill_layer_gpu(cfg, h, slot, wk, wv, len(layers), parts, pos=pos, row_idx=rows.to(DEV),
                            m_dev=m_dev, m_max=64)
    check_layer(cfg, kc, vc, h, sel.numpy(), slot, None, wk, wv, parts, pos)


@pytest.mark.parametrize("norm,bias,rope", [(True, True, True), (False, False, True),
                                            (False, True, False), (True, False, False)])
def test_layer_fill_parts_with_maps(norm, bias, rope):
    """Each part alone and all together, with maps (Llama-3.2-1B shape)."""
    cfg = get_config(2)
    layers = list(range(9, 13))
    h = G.hidden_states(cfg, cfg.n_tokens, [8])[8].to(DEV)
    slot = G.slots(cfg, device=DEV)
    pos = slot.clone()
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, len(layers)).to(DEV)
    parts = _parts(cfg, layers, norm, bias, rope)
    rows = torch.tensor([5, 0, 63, 17, 33, 2], dtype=torch.int32, device=DEV)
    kc, vc = fill_layer_gpu(cfg, h, slot, wk, wv, len(layers), parts, pos=pos, row_idx=rows,
                            maps=maps)
    check_layer(cfg, kc, vc, h, rows.cpu().numpy(), slot, maps, wk, wv, parts, pos)


@pytest.mark.parametrize("ws_layers,gemm_path", [(8, 0), (3, 0), (8, 2)])
def test_layer_fill_gpt2_ridge_maps_norm_bias(ws_layers, gemm_path):
    """GPT-2-shape prefill: ridge maps, input RMSNorm and K/V biases (no
    rotary embedding), half of the 4096 tokens, count on the device; with
    gemm_path 2 the map GEMM (with its RMSNorm epilogue) runs on 256 x 256
    tiles."""
    tee.river_debug_set_gemm_path(gemm_path)
    try:
        _gpt2_ridge_maps_norm_bias(ws_layers)
    finally:
        tee.river_debug_set_gemm_path(0)


def _gpt2_ridge_maps_norm_bias(ws_layers):
    cfg = get_config(1)
    e = 4
    layers = list(range(e + 1, cfg.L + 1))
    X, Y = G.calibration(cfg, e)
    maps = torch.from_numpy(O.ridge_fit(np64(X), np64(Y), cfg.ridge_lambda)).bfloat16().to(DEV)
    h = G.hidden_states(cfg, cfg.n_tokens, [e])[e].to(DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers)
    parts = _parts(cfg, layers, rope=False)
    g = torch.Generator().manual_seed(7)
    sel = torch.nonzero(torch.rand(cfg.n_tokens, generator=g) < 0.5).flatten().to(torch.int32)
    rows = torch.full((cfg.n_tokens,), -1, dtype=torch.int32)
    rows[: sel.numel()] = sel
    m_dev = torch.tensor([sel.numel()], dtype=torch.int32, device=DEV)
    kc, vc = fill_layer_gpu(cfg, h, slot, wk, wv, len(layers), parts, row_idx=rows.to(DEV),
                            m_dev=m_dev, m_max=cfg.n_tokens, maps=maps, ws_layers=ws_layers)
    pick = np.sort(np.random.default_rng(5).choice(sel.numel(), 128, replace=False))
    check_layer(cfg, kc, vc, h, sel.numpy(), slot, maps, wk, wv, parts, None, sample=pick)


def test_layer_fill_8b_prefill_sampled():
    """Llama-3-8B-shape prefill: 410 exits of 8192 tokens, maps, input
    RMSNorm and RoPE (head_dim 128) at the token positions."""
    cfg = get_config(3)
    e = 11
    layers = list(range(e + 1, cfg.L + 1))
    h = G.hidden_states(cfg, cfg.n_tokens, [e], device=DEV)[e]
    slot = G.slots(cfg, device=DEV)
    pos = torch.arange(cfg.n_tokens, dtype=torch.int32, device=DEV)
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, len(layers), device=DEV)
    parts = _parts(cfg, layers, bias=False, n_pos=cfg.n_tokens)
    g = torch.Generator().manual_seed(13)
    sel = torch.sort(torch.randperm(cfg.n_tokens, generator=g)[:410]).values.to(torch.int32)
    kc, vc = fill_layer_gpu(cfg, h, slot, wk, wv, len(layers), parts, pos=pos,
                            row_idx=sel.to(DEV), maps=maps)
    pick = np.sort(np.random.default_rng(6).choice(410, 16, replace=False))
    check_layer(cfg, kc, vc, h, sel.numpy(), slot, maps, wk, wv, parts, pos, sample=pick)


@pytest.mark.parametrize("cfg_idx,over", [
    (0, {}),                                                   # fp32: generic kernel
    (1, dict(d=200, n_kv_heads=3, head_dim=24, group=40, n_tokens=40, n_slots=96)),
    (2, dict(head_dim=48, n_kv_heads=4)),                      # head_dim % 32 != 0 with RoPE
])
def test_layer_fill_generic_shapes(cfg_idx, over):
    cfg = get_config(cfg_idx, **over)
    layers = [3, 4, 5]
    h = G.hidden_states(cfg, cfg.n_tokens, [2])[2].to(DEV)
    gen = torch.Generator().manual_seed(cfg.d)
    slot = torch.randperm(cfg.n_slots, generator=gen)[: cfg.n_tokens].to(torch.int32).to(DEV)
    pos = torch.randint(0, 300, (cfg.n_tokens,), generator=gen, dtype=torch.int32).to(DEV)
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, len(layers)).to(DEV)
    parts = _parts(cfg, layers, n_pos=300)
    rows = torch.tensor([1, 7, 0, 22, 39], dtype=torch.int32, device=DEV)
    for mp in (None, maps):
        kc, vc = fill_layer_gpu(cfg, h, slot, wk, wv, len(layers), parts, pos=pos, row_idx=rows,
                                maps=mp)
        check_layer(cfg, kc, vc, h, rows.cpu().numpy(), slot, mp, wk, wv, parts, pos)


def test_layer_fill_position_out_of_table_is_skipped():
    cfg = get_config(2)
    layers = [9, 10]
    h = G.hidden_states(cfg, cfg.n_tokens, [8])[8].to(DEV)
    slot = G.slots(cfg, device=DEV)
    pos = torch.arange(cfg.n_tokens, dtype=torch.int32)
    pos[3] = 5000                               # past the 4096-row table
    pos[10] = -1
    pos = pos.to(DEV)
    wk, wv = _kv(cfg, layers)
    parts = _parts(cfg, layers, bias=False)
    rows = torch.tensor([2, 3, 10, 11], dtype=torch.int32, device=DEV)
    for mp in (None, G.near_identity_maps(cfg, len(layers)).to(DEV)):
        kc, vc = fill_layer_gpu(cfg, h, slot, wk, wv, len(layers), parts, pos=pos, row_idx=rows,
                                maps=mp)
        check_layer(cfg, kc, vc, h, rows.cpu().numpy(), slot, mp, wk, wv, parts, pos,
                    skipped=(3, 10))


def test_layer_fill_with_nothing_on_equals_kv_fill():
    cfg = get_config(1)
    layers = list(range(5, 13))
    h = G.hidden_states(cfg, cfg.n_tokens, [4])[4].to(DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, layers)
    maps = G.near_identity_maps(cfg, len(layers)).to(DEV)
    rows = torch.arange(0, cfg.n_tokens, 7, dtype=torch.int32, device=DEV)
    k1, v1 = fill_layer_gpu(cfg, h, slot, wk, wv, len(layers), {}, row_idx=rows, maps=maps)
    k2 = torch.full_like(k1, float("nan"))
    v2 = torch.full_like(v1, float("nan"))
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, rows.numel(), cfg.d, 0, 0, len(layers)),
                     dtype=torch.uint8, device=DEV)
    tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, k2, v2, row_idx=rows, maps=maps,
                      workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
