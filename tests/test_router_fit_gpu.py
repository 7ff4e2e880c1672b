"""GPU parity of router calibration (river_router_fit, labels through
river_route) against the float64 oracle.

Bars:
* labels (river_route, router off, tau = 0.98) bit-exact outside the 1e-4
  band around the threshold;
* one Adam step: the GPU's update of every parameter within 1e-3 lr of the
  oracle's, for parameters whose gradient the oracle puts well above Adam's
  eps (its update at least 0.99 lr; below that the update's size depends on
  the gradient's last digits, which fp32 does not resolve);
* a whole fit (100 epochs of 8 shuffled mini-batches, 800 Adam steps):
  final weights within 1e-4 of the total update (relative Frobenius of the
  difference to the oracle over the oracle's change from the start), the
  mean loss of every epoch within 1e-6 plus 1e-3 of itself, the same
  calibration-set decisions for all but 0.1% of the tokens;
* two fits give the same bits.
Derivation of the whole-fit bar: each step's fp32 gradient carries a
relative error of order the fp32 unit roundoff (6e-8) and Adam moves every
resolved parameter by a bounded step, so if every step's error added up
with no cancellation the weights would drift by at most 800 x 6e-8 = 4.8e-5
of the total update; 1e-4 rounds that up (measured: 1.2e-6).
"""

import numpy as np
import pytest
import torch

import oracle as O
import token_early_exit_amd as tee
from synth import get_config
from synth import generate as G
from helpers import BAND, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


def labels_gpu(hk, hf):
    mask = torch.empty(hk.shape[0], dtype=torch.uint8, device=DEV)
    cos = torch.empty(hk.shape[0], device=DEV)
    tee.river_route(hf, hk, mask, tau=0.98, cos_out=cos)
    torch.cuda.synchronize()
    return mask, cos


def fit_gpu(h, y, W0, w0, epochs, batch, order=None, lr=1e-3):
    W = torch.tensor(W0, dtype=torch.float32, device=DEV)
    w = torch.tensor(w0, dtype=torch.float32, device=DEV)
    loss = torch.full((epochs,), float("nan"), device=DEV)
    n, d = h.shape
    ws = torch.empty(tee.river_workspace_size(tee.OP_ROUTER_FIT, n, d, W.shape[0], batch, epochs),
                     dtype=torch.uint8, device=DEV)
    tee.river_router_fit(h, y, W, w, epochs=epochs, batch=batch, order=order, lr=lr,
                         loss_out=loss, workspace=ws)
    torch.cuda.synchronize()
    return W, w, loss


def _case(n=None):
    cfg = get_config(1)
    hk, hf = G.router_calibration(cfg, 4, n)
    hk, hf = hk.to(DEV), hf.to(DEV)
    wd, wu = G.router_weights(cfg, 4)
    return cfg, hk, hf, wd.float().numpy().astype(np.float64), wu.float().numpy().astype(np.float64)


def test_router_labels_from_route():
    cfg, hk, hf, _, _ = _case()
    mask, cos = labels_gpu(hk, hf)
    ref = O.router_labels(np64(hk), np64(hf), 0.98)
    c, *_ = O.route(np64(hf), np64(hk), None, 0.0, None, None, -np.inf, -np.inf)
    band = np.abs(c - np.float32(0.98)) < BAND
    assert np.array_equal(mask.cpu().numpy()[~band], ref[~band])
    assert 0.3 < ref.mean() < 0.55 and band.sum() <= 5


def test_router_fit_one_step():
    cfg, hk, hf, W0, w0 = _case(1000)
    y, _ = labels_gpu(hk, hf)
    lr = 1e-3
    W, w, loss = fit_gpu(hk, y, W0, w0, 1, 1000, lr=lr)
    Wr, wr, lr_ = O.router_fit(np64(hk), y.cpu().numpy(), W0, w0, 1, 1000, lr=lr)
    for got, ref, start in ((W, Wr, W0), (w, wr, w0)):
        dg = got.cpu().double().numpy() - start
        dr = ref - start
        sure = np.abs(dr) >= 0.99 * lr
        assert sure.mean() > 0.95
        assert np.all(np.abs(dg[sure] - dr[sure]) <= 1e-3 * lr)
        assert np.all(np.abs(dg) <= lr * (1 + 1e-5))          # Adam's first step is at most lr
    assert abs(loss.item() - lr_[0]) <= 1e-5


def test_router_fit_whole_fit_shuffled():
    cfg, hk, hf, W0, w0 = _case()
    n = hk.shape[0]
    y, _ = labels_gpu(hk, hf)
    epochs, batch = 100, 256
    rng = np.random.default_rng(8)
    order = np.stack([rng.permutation(n) for _ in range(epochs)]).astype(np.int32)
    W, w, loss = fit_gpu(hk, y, W0, w0, epochs, batch, torch.from_numpy(order).to(DEV))
    yn = y.cpu().numpy()
    Wr, wr, lr_ = O.router_fit(np64(hk), yn, W0, w0, epochs, batch, order)
    lg = loss.cpu().double().numpy()
    assert np.all(np.abs(lg - lr_) <= 1e-6 + 1e-3 * lr_), np.abs(lg - lr_).max()
    assert lr_[-1] < 0.1 * lr_[0]                            # it learns
    Wg = W.cpu().double().numpy()
    wg = w.cpu().double().numpy()
    rel = np.linalg.norm(Wg - Wr) / np.linalg.norm(Wr - W0)
    relw = np.linalg.norm(wg - wr) / np.linalg.norm(wr - w0)
    assert rel <= 1e-4 and relw <= 1e-4, (rel, relw)
    h = np64(hk)
    _, pg, _, _ = O.route(h, h, None, 1e-6, Wg, wg, -np.inf, -np.inf)
    _, pr, _, _ = O.route(h, h, None, 1e-6, Wr, wr, -np.inf, -np.inf)
    assert np.mean((pg > 0.5) != (pr > 0.5)) <= 0.001


def test_router_fit_ragged_last_batch_and_determinism():
    cfg, hk, hf, W0, w0 = _case(1000)
    y, _ = labels_gpu(hk, hf)
    W1, w1, l1 = fit_gpu(hk, y, W0, w0, 3, 96)           # 10 batches of 96 and one of 40
    W2, w2, l2 = fit_gpu(hk, y, W0, w0, 3, 96)
    assert torch.equal(W1, W2) and torch.equal(w1, w2) and torch.equal(l1, l2)
    Wr, wr, lr_ = O.router_fit(np64(hk), y.cpu().numpy(), W0, w0, 3, 96)
    assert np.all(np.abs(l1.cpu().double().numpy() - lr_) <= 1e-6 + 1e-4 * lr_)
    rel = np.linalg.norm(W1.cpu().double().numpy() - Wr) / np.linalg.norm(Wr - W0)
    assert rel <= 1e-4, rel


@pytest.mark.parametrize("dt,b,d", [(torch.float32, 200, 264), (torch.bfloat16, 320, 136),
                                    (torch.bfloat16, 96, 520)])
def test_router_fit_shapes_with_gamma(dt, b, d):
    """Unit counts that are not multiples of 128 (several unit groups per
    thread), feature counts that leave ragged chunks, fp32 states and a
    router RMSNorm weight."""
    g = torch.Generator().manual_seed(b + d)
    n = 300
    h = (torch.randn(n, d, generator=g) * torch.rand(n, 1, generator=g).add(0.5)).to(dt)
    v = torch.randn(d, generator=g)
    y = ((h.float() @ v) > 0).to(torch.uint8)
    gam = (1 + 0.1 * torch.randn(d, generator=g)).to(dt)
    W0 = (torch.randn(b, d, generator=g) / d ** 0.5).double().numpy()
    w0 = (torch.randn(b, generator=g) / b ** 0.5).double().numpy()
    hd, yd, gd = h.to(DEV), y.to(DEV), gam.to(DEV)
    W = torch.tensor(W0, dtype=torch.float32, device=DEV)
    w = torch.tensor(w0, dtype=torch.float32, device=DEV)
    loss = torch.empty(4, device=DEV)
    ws = torch.empty(tee.river_workspace_size(tee.OP_ROUTER_FIT, n, d, b, 64, 4), dtype=torch.uint8,
                     device=DEV)
    tee.river_router_fit(hd, yd, W, w, epochs=4, batch=64, gamma=gd, eps=1e-5, lr=3e-3,
                         loss_out=loss, workspace=ws)
    torch.cuda.synchronize()
    Wr, wr, lr_ = O.router_fit(np64(h), y.numpy(), W0, w0, 4, 64, gamma=np64(gam), eps=np.float32(1e-5),
                               lr=np.float32(3e-3))
    rel = np.linalg.norm(W.cpu().double().numpy() - Wr) / np.linalg.norm(Wr - W0)
    relw = np.linalg.norm(w.cpu().double().numpy() - wr) / np.linalg.norm(wr - w0)
    assert rel <= 1e-4 and relw <= 1e-4, (rel, relw)
    assert np.all(np.abs(loss.cpu().double().numpy() - lr_) <= 1e-6 + 1e-4 * lr_)
