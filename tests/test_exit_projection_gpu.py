"""GPU parity of the exit projection (final RMSNorm of the exited rows,
scattered to their row ids) against the float64 oracle.

Bar, element by element against the oracle's float64 value o:
* bf16 output: |gpu - o| <= 2^-8 |o|. The kernel's fp32 arithmetic is
  within about 1e-5 relative of o and rounding to bf16 adds at most half an
  ulp (2^-9 relative), so one bf16 ulp bounds the sum.
* fp32 output: |gpu - o| <= 1e-5 |o| + 1e-6 max_j |o_j| (fp32 sum of
  squares over at most 16384 terms, one reciprocal square root, two
  products).
Rows that receive nothing keep their NaN sentinel bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import token_early_exit_amd as tee
from synth import get_config
from synth import generate as G
from helpers import np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


def check(out_gpu, ref):
    """out_gpu: device tensor [N][d]; ref: float64 oracle output [N][d]."""
    o = out_gpu.cpu().double().numpy()
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(o), nan_ref)
    rows = ~nan_ref.all(axis=1)
    a, b = o[rows], ref[rows]
    if out_gpu.dtype == torch.bfloat16:
        tol = 2.0 ** -8 * np.abs(b)
    else:
        tol = 1e-5 * np.abs(b) + 1e-6 * np.abs(b).max(axis=1, keepdims=True)
    err = np.abs(a - b)
    assert np.all(err <= tol), float((err - tol).max())
    return int(rows.sum())


def project_gpu(h, out, **kw):
    tee.river_exit_projection(h, out, **kw)
    torch.cuda.synchronize()
    return out


def _rand(n, d, dt, seed, scale=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, d, generator=g)
    if scale is not None:
        x *= torch.exp(torch.randn(n, 1, generator=g) * scale)
    return x.to(dt)


def test_exit_projection_gpt2_after_compact():
    """route -> compact -> exit projection on the GPT-2-shape prefill batch,
    the exit count and rows passed on the device."""
    cfg = get_config(1)
    e = 4
    n, d = cfg.n_tokens, cfg.d
    hs = {l: t.to(DEV) for l, t in G.hidden_states(cfg, n, [e - 1, e]).items()}
    wd, wu = (t.to(DEV) for t in G.router_weights(cfg, e))
    gamma = G.final_norm_gamma(cfg).to(DEV)
    g = torch.Generator().manual_seed(5)
    n_total = 2 * n
    rid = torch.randperm(n_total, generator=g)[:n].to(torch.int32).to(DEV)
    mask = torch.empty(n, dtype=torch.uint8, device=DEV)
    tee.river_route(hs[e - 1], hs[e], mask, w_down=wd, w_up=wu, tau=cfg.tau, theta=cfg.theta)
    cont = torch.empty(n, dtype=torch.int32, device=DEV)
    ext = torch.empty(n, dtype=torch.int32, device=DEV)
    counts = torch.empty(2, dtype=torch.int32, device=DEV)
    ws = torch.empty(tee.river_workspace_size(tee.OP_COMPACT, n), dtype=torch.uint8, device=DEV)
    tee.river_compact(mask, hs[e], cont, ext, counts, row_ids=rid, workspace=ws)
    out = torch.full((n_total, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    project_gpu(hs[e], out, m_max=n, m_dev=counts[1:], row_idx=ext, row_ids=rid, gamma=gamma,
                eps=1e-5)
    c = O.compact(mask.cpu().numpy(), None)
    ne = int(c["counts"][1])
    assert 0 < ne < n
    ref = O.exit_projection(np64(hs[e]), c["exit_idx"], ne, np64(gamma), np.float32(1e-5),
                            np.full((n_total, d), np.nan), rid.cpu().numpy())
    assert check(out, ref) == ne


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [8, 72, 256, 768, 1032, 2048, 4096, 4104, 8192, 8200, 16384])
def test_exit_projection_widths(dt, d):
    """Every register-resident chunk count and the streamed variant, with
    ragged last chunks, gamma, a permuted scatter and rows of very different
    scale."""
    n = 67
    h = _rand(n, d, dt, seed=d, scale=3.0).to(DEV)
    gamma = (1 + 0.1 * torch.randn(d, generator=torch.Generator().manual_seed(d + 1))).to(dt).to(DEV)
    g = torch.Generator().manual_seed(d + 2)
    rows = torch.randperm(n, generator=g)[:45].to(torch.int32).to(DEV)
    rid = torch.randperm(n + 9, generator=g)[:n].to(torch.int32).to(DEV)
    out = torch.full((n + 9, d), float("nan"), dtype=dt, device=DEV)
    project_gpu(h, out, row_idx=rows, row_ids=rid, gamma=gamma, eps=1e-6)
    ref = O.exit_projection(np64(h), rows.cpu().numpy(), 45, np64(gamma), np.float32(1e-6),
                            np.full((n + 9, d), np.nan), rid.cpu().numpy())
    assert check(out, ref) == 45


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_exit_projection_edges(dt):
    d = 136
    n = 12
    h = _rand(n, d, dt, seed=77).to(DEV)
    h[5] = 0
    full = lambda rows: torch.full((rows, d), float("nan"), dtype=dt, device=DEV)
    nan_ref = lambda rows: np.full((rows, d), np.nan)
    # m_max = 0: nothing written
    out = full(n)
    project_gpu(h, out, m_max=0)
    assert torch.isnan(out).all()
    # device count: 0, negative, above m_max (clamped), inside
    for m_dev, m_max, rows_done in ((0, 10, 0), (-3, 10, 0), (50, 7, 7), (4, 10, 4)):
        md = torch.tensor([m_dev], dtype=torch.int32, device=DEV)
        out = full(n)
        project_gpu(h, out, m_max=m_max, m_dev=md)
        ref = O.exit_projection(np64(h), None, rows_done, None, np.float32(1e-6), nan_ref(n))
        assert check(out, ref) == rows_done
    # no gamma, eps = 0: a zero row gives NaN, every other row unit RMS
    out = full(n)
    project_gpu(h, out, eps=0.0)
    ref = O.exit_projection(np64(h), None, n, None, 0.0, nan_ref(n))
    ok = np.ones(n, bool)
    ok[5] = False
    assert torch.isnan(out[5]).all()
    o = out.cpu().double().numpy()
    assert np.all(np.abs(o[ok] - ref[ok]) <= 2.0 ** -8 * np.abs(ref[ok]) + 1e-30)
    # out-of-range rows and destinations are skipped; a short output
    rows = torch.tensor([3, -1, n, 7, 9, 11], dtype=torch.int32, device=DEV)
    rid = torch.arange(n, dtype=torch.int32, device=DEV).flip(0).contiguous()
    rid[9] = 40
    rid[11] = -2
    out = full(9)
    project_gpu(h, out, row_idx=rows, row_ids=rid, eps=1e-3)
    ref = O.exit_projection(np64(h), rows.cpu().numpy(), 6, None, np.float32(1e-3), nan_ref(9),
                            rid.cpu().numpy())
    assert check(out, ref) == 2          # rows 3 and 7 land at 8 and 4
    # strided input and output (leading dims above d)
    hb = _rand(n, d + 24, dt, seed=78).to(DEV)
    ob = torch.full((n, d + 40), float("nan"), dtype=dt, device=DEV)
    project_gpu(hb[:, :d], ob[:, :d], eps=1e-6)
    ref = O.exit_projection(np64(hb[:, :d]), None, n, None, np.float32(1e-6), nan_ref(n))
    assert check(ob[:, :d], ref) == n
    assert torch.isnan(ob[:, d:]).all()


def test_exit_projection_8b_prefill_sampled():
    """Llama-3-8B-shape prefill width (d = 4096, 8192 tokens), every row of
    the batch projected through a permutation; sampled rows checked."""
    cfg = get_config(3)
    n, d = cfg.n_tokens, cfg.d
    h = G.hidden_states(cfg, n, [cfg.route_layers[0]])[cfg.route_layers[0]].to(DEV)
    gamma = G.final_norm_gamma(cfg).to(DEV)
    g = torch.Generator().manual_seed(9)
    rid = torch.randperm(n, generator=g).to(torch.int32).to(DEV)
    out = torch.full((n, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    project_gpu(h, out, row_ids=rid, gamma=gamma, eps=1e-5)
    pick = np.sort(np.random.default_rng(3).choice(n, 256, replace=False))
    hp = np64(h[torch.from_numpy(pick).to(DEV)])
    ref = O.exit_projection(hp, None, len(pick), np64(gamma), np.float32(1e-5),
                            np.zeros((len(pick), d)))
    dst = rid.cpu().numpy()[pick]
    o = out[torch.from_numpy(dst).long().to(DEV)].cpu().double().numpy()
    assert np.all(np.abs(o - ref) <= 2.0 ** -8 * np.abs(ref))
    assert not torch.isnan(out).any()         # a permutation fills every row
