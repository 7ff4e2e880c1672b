"""Comparison helpers for the GPU parity tests (they may call the oracle)."""

import math

import numpy as np
import torch

import oracle as O

BAND = 1e-4        # tokens this close to a threshold are excluded from mask checks
COS_TOL = 2e-3     # |d cos|, |d prob|
KV_TOL = 1e-2      # per-row relative L2 error of K and V


def np64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def f32(x):
    """A threshold as the kernel sees it (an fp32 argument)."""
    return float(np.float32(x))


def check_route(gpu, ref, tau, theta, router, rule=O.RULE_TOKEN):
    """gpu: (cos, prob, mask, all_exit) tensors; ref: oracle tuple.
    Returns the number of tokens excluded by the threshold band."""
    gcos, gprob, gmask, gall = [t.cpu() for t in gpu]
    ocos, oprob, omask, oall = ref
    gc = gcos.numpy()
    gp = gprob.numpy()
    gm = gmask.numpy()
    both = np.isfinite(ocos)
    assert np.array_equal(np.isnan(gc), np.isnan(ocos))
    assert np.all(np.abs(gc[both] - ocos[both]) <= COS_TOL), np.max(np.abs(gc[both] - ocos[both]))
    if router:
        fin = np.isfinite(oprob)
        assert np.all(np.abs(gp[fin] - oprob[fin]) <= COS_TOL), np.max(np.abs(gp[fin] - oprob[fin]))
    else:
        assert np.all(gp == 1.0)
    # the kernel's decision, taken in fp32 on its own fp32 values
    with np.errstate(invalid="ignore"):
        own = (gc > np.float32(tau)) & ((gp > np.float32(theta)) if router else True)
    band = np.abs(ocos - tau) < BAND
    if router:
        band |= np.abs(oprob - theta) < BAND
    band &= np.isfinite(ocos)
    if rule == O.RULE_TOKEN:
        assert np.array_equal(gm, own.astype(np.uint8))
        assert np.array_equal(gm[~band], omask[~band])
        assert int(gall) == int(own.size > 0 and bool(np.all(own)))
    else:
        a = int(own.size > 0 and bool(np.all(own)))
        assert int(gall) == a and np.all(gm == a)
        if not band.any():
            assert a == oall
    return int(band.sum())


def kv_row_errors(gpu_rows, ref_rows):
    """Per-row relative L2 error, rows along the last axis."""
    g = np64(gpu_rows).reshape(-1, gpu_rows.shape[-1])
    r = np64(ref_rows).reshape(-1, ref_rows.shape[-1])
    num = np.linalg.norm(g - r, axis=1)
    den = np.maximum(np.linalg.norm(r, axis=1), 1e-6)
    return num / den


def w4_np(w):
    q, s, z, group = w
    return {"q": q.cpu().numpy(), "scale": np64(s), "zero": np64(z), "group": group}


def midpoint_threshold(values, k_from_top):
    """Threshold between the k-th and (k+1)-th largest values."""
    v = np.sort(values)[::-1]
    return 0.5 * (v[k_from_top - 1] + v[k_from_top])


def inf():
    return math.inf
