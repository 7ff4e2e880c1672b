"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these retypes the oracle's own formula: each checks an identity, a
worked example the pages print, a hand-worked value, a library routine that
implements the same definition independently, or brute force on tiny
inputs. A plausible slip in the oracle (a dropped term, a wrong sign or
index, a transposed operand) fails at least one of them; the mutation tests
at the end plant such slips in a copy of the oracle and check that.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- P1 cosine

def test_p1_cosine_identities():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((50, 33))
    cos, *_ = O.route(a, a, None, 1e-6, None, None, -np.inf, -np.inf)
    assert np.all(cos == 1.0)                       # cos(a, a) = 1 exactly
    cos, *_ = O.route(a, -a, None, 1e-6, None, None, -np.inf, -np.inf)
    assert np.all(cos == -1.0)                      # cos(a, -a) = -1
    k = rng.uniform(0.1, 10.0, size=(50, 1))
    cos, *_ = O.route(a, k * a, None, 1e-6, None, None, -np.inf, -np.inf)
    assert np.allclose(cos, 1.0, atol=1e-15, rtol=0)
    # orthogonal pair
    x = np.zeros((2, 4)); y = np.zeros((2, 4))
    x[0, 0] = 3.0; y[0, 1] = -2.0
    x[1] = [1, 1, 0, 0]; y[1] = [1, -1, 5, 0]
    cos, *_ = O.route(x, y, None, 1e-6, None, None, -np.inf, -np.inf)
    assert np.all(cos == 0.0)
    # zero vector: defined as 0; NaN input: NaN cosine, never exits
    z = np.zeros((1, 4)); w = np.array([[1.0, 2.0, 3.0, np.nan]])
    cos, _, mask, _ = O.route(z, z + 1, None, 1e-6, None, None, -np.inf, -np.inf)
    assert cos[0] == 0.0
    cos, _, mask, _ = O.route(w, w, None, 1e-6, None, None, -np.inf, -np.inf)
    assert np.isnan(cos[0]) and mask[0] == 0


def test_p1_cosine_matches_scipy_and_bounds():
    from scipy.spatial.distance import cdist
    rng = np.random.default_rng(2)
    a = rng.standard_normal((100_000, 8))
    b = rng.standard_normal((100_000, 8)) * rng.uniform(0.01, 100, (100_000, 1))
    cos, *_ = O.route(a, b, None, 1e-6, None, None, -np.inf, -np.inf)
    assert np.all(cos <= 1.0) and np.all(cos >= -1.0)         # Cauchy-Schwarz
    ref = 1.0 - np.array([cdist(a[i:i + 1], b[i:i + 1], "cosine")[0, 0] for i in range(200)])
    assert np.allclose(cos[:200], ref, atol=1e-12, rtol=0)


# ------------------------------------------------------- P2 the schedule

def test_p2_tide_figure2_worked_example():
    g = _gold("tide_fig2_schedule.json")
    r = O.exit_schedule_ops(g["exit_layers"], g["n_layers"])
    assert r["executed"] == g["executed"] == 56
    assert r["baseline"] == g["baseline"] == 96
    assert round(100 * r["reduction"]) == g["reduction_percent_rounded"]
    # every skipped (token, layer) is filled: executed + filled = baseline
    assert r["filled"] == 40 and r["executed"] + r["filled"] == r["baseline"]
    with pytest.raises(ValueError):
        O.exit_schedule_ops([0], 32)


# ------------------------------------------------------------ P3 ridge

def _ridge_obj(X, Y, W, lam):
    # W in output-major layout [d_out][d_in]
    R = X @ W.T - Y
    return float(np.sum(R * R) + lam * np.sum(W * W))


def test_p3_ridge_normal_equations_and_orientation():
    rng = np.random.default_rng(3)
    n, d_in, d_out, T = 40, 7, 5, 3
    X = rng.standard_normal((n, d_in))
    Y = rng.standard_normal((T, n, d_out))
    lam = 0.3
    W = O.ridge_fit(X, Y, lam)
    assert W.shape == (T, d_out, d_in)
    G = X.T @ X + lam * np.eye(d_in)
    for t in range(T):
        res = G @ W[t].T - X.T @ Y[t]
        assert np.linalg.norm(res) <= 1e-10 * np.linalg.norm(X.T @ Y[t])


def test_p3_ridge_matches_lstsq_and_sklearn():
    from sklearn.linear_model import Ridge
    rng = np.random.default_rng(4)
    n, d = 64, 8
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((2, n, 3))
    # lambda -> 0 on a full-rank system: ordinary least squares
    W = O.ridge_fit(X, Y, 1e-12)
    for t in range(2):
        ls = np.linalg.lstsq(X, Y[t], rcond=None)[0]       # [d_in][d_out]
        assert np.allclose(W[t], ls.T, atol=1e-9)
    # an independent ridge implementation, no intercept
    W = O.ridge_fit(X, Y, 2.5)
    for t in range(2):
        sk = Ridge(alpha=2.5, fit_intercept=False, solver="svd").fit(X, Y[t])
        assert np.allclose(W[t], sk.coef_, atol=1e-10)


def test_p3_ridge_closed_forms():
    rng = np.random.default_rng(5)
    n, d = 50, 6
    X = rng.standard_normal((n, d))
    Wstar = rng.standard_normal((4, d))                       # output-major
    # exact linear targets, lambda = 0: the map is recovered
    W = O.ridge_fit(X, (X @ Wstar.T)[None], 0.0)
    assert np.allclose(W[0], Wstar, atol=1e-10)
    # Y = X: W = I - lambda (X^T X + lambda I)^-1
    lam = 0.7
    W = O.ridge_fit(X, X[None], lam)
    G = X.T @ X + lam * np.eye(d)
    assert np.allclose(W[0], np.eye(d) - lam * np.linalg.inv(G), atol=1e-12)
    # lambda -> infinity: W -> 0, bounded by |X^T Y| / lambda
    Y = rng.standard_normal((1, n, 3))
    W = O.ridge_fit(X, Y, 1e12)
    assert np.linalg.norm(W) <= np.linalg.norm(X.T @ Y[0]) / 1e12 * 1.0001


def test_p3_ridge_brute_force_minimum():
    rng = np.random.default_rng(6)
    X = rng.standard_normal((12, 3))
    Y = rng.standard_normal((1, 12, 2))
    lam = 0.5
    W = O.ridge_fit(X, Y, lam)[0]
    f0 = _ridge_obj(X, Y[0], W, lam)
    for _ in range(2000):
        P = rng.standard_normal(W.shape) * rng.choice([1e-1, 1e-3, 1e-5])
        assert _ridge_obj(X, Y[0], W + P, lam) >= f0 - 1e-12


# ---------------------------------------------------------- P4 compaction

def _check_partition(mask, res, h):
    n = len(mask)
    cont, ext = list(res["cont_idx"]), list(res["exit_idx"])
    assert set(cont).isdisjoint(ext)
    assert sorted(cont + ext) == list(range(n))
    assert cont == sorted(cont) and ext == sorted(ext)
    assert all(mask[i] == 0 for i in cont) and all(mask[i] != 0 for i in ext)
    assert list(res["counts"]) == [len(cont), len(ext)]
    if h is not None:
        for j, i in enumerate(cont):
            assert np.array_equal(res["h_cont"][j], h[i])


def test_p4_compaction_exhaustive_small():
    for n in range(0, 13):
        h = np.arange(n * 2, dtype=np.float64).reshape(n, 2)
        for bits in range(1 << n):
            mask = np.array([(bits >> i) & 1 for i in range(n)], dtype=np.uint8)
            _check_partition(mask, O.compact(mask, h), h)


@pytest.mark.parametrize("n", [0, 1, 63, 64, 65, 1023, 1024, 1025, 8192])
def test_p4_compaction_edges(n):
    rng = np.random.default_rng(n)
    h = rng.standard_normal((n, 3))
    rid = rng.permutation(4 * n + 1)[:n] if n else np.zeros(0, dtype=np.int64)
    out = np.full((4 * n + 1, 3), np.nan)
    for mask in (np.zeros(n, np.uint8), np.ones(n, np.uint8),
                 (rng.random(n) < 0.3).astype(np.uint8)):
        res = O.compact(mask, h, rid, out)
        _check_partition(mask, res, h)
        assert np.array_equal(res["row_ids_cont"], rid[res["cont_idx"]])
        # exit scatter: exited rows land at their row id, nothing else moves
        o = res["out"]
        hit = set(int(rid[i]) for i in res["exit_idx"])
        for i in res["exit_idx"]:
            assert np.array_equal(o[rid[i]], h[i])
        for r in range(o.shape[0]):
            if r not in hit:
                assert np.all(np.isnan(o[r]))


# ------------------------------------------------------------- P5 kv fill

def _hand_w4(n_layers, n_out, d, group, rng):
    q = rng.integers(0, 256, size=(n_layers, n_out, d // 2), dtype=np.uint8)
    s = rng.uniform(0.01, 0.1, size=(n_layers, n_out, d // group))
    z = rng.uniform(0, 15, size=(n_layers, n_out, d // group))
    return {"q": q, "scale": s, "zero": z, "group": group}


def test_p5_identity_fill_is_direct_projection():
    rng = np.random.default_rng(7)
    d, Hkv, Dh, nl = 16, 2, 4, 3
    wk = _hand_w4(nl, Hkv * Dh, d, 8, rng)
    wv = _hand_w4(nl, Hkv * Dh, d, 8, rng)
    # one-hot rows: the projection of e_k is column k of the dequantized weights
    h = np.eye(d)[[3, 0, 11, 15]]
    K, V = O.kv_fill_rows(h, None, 4, None, wk, wv)
    Ke, Ve = O.kv_fill_rows(h, None, 4, np.stack([np.eye(d)] * nl), wk, wv)
    assert np.array_equal(K, Ke) and np.array_equal(V, Ve)
    for l in range(nl):
        Wk = O.dequant_w4(wk["q"][l], wk["scale"][l], wk["zero"][l], 8)
        for t, k in enumerate([3, 0, 11, 15]):
            # hand unpack of element k of every output row
            byte = wk["q"][l][:, k // 2]
            nib = (byte & 15) if k % 2 == 0 else (byte >> 4)
            want = (nib - wk["zero"][l][:, k // 8]) * wk["scale"][l][:, k // 8]
            assert np.allclose(K[l, t], want, rtol=0, atol=1e-15)
            assert np.allclose(Wk[:, k], want, rtol=0, atol=1e-15)


def test_p5_map_orientation_and_slots():
    rng = np.random.default_rng(8)
    d, Hkv, Dh, nl = 8, 2, 2, 2
    wk = _hand_w4(nl, Hkv * Dh, d, 4, rng)
    wv = _hand_w4(nl, Hkv * Dh, d, 4, rng)
    perm = [rng.permutation(d) for _ in range(nl)]
    maps = np.zeros((nl, d, d))
    for l in range(nl):
        for j in range(d):
            maps[l, j, perm[l][j]] = 1.0      # x_hat[j] = x[perm[j]]
    h = rng.standard_normal((5, d))
    row_idx = np.array([4, 1, 2])
    slot = np.array([9, 3, 0, 7, 5])           # slot of each row of h
    kc0 = np.full((nl, 10, Hkv, Dh), np.nan)
    kc, vc = O.kv_fill(h, row_idx, 3, slot, maps, wk, wv, Hkv, Dh, kc0, kc0)
    for l in range(nl):
        Wk = O.dequant_w4(wk["q"][l], wk["scale"][l], wk["zero"][l], 4)
        for t, r in enumerate(row_idx):
            xh = h[r][perm[l]]
            want = np.array([sum(Wk[o, j] * xh[j] for j in range(d)) for o in range(Hkv * Dh)])
            assert np.allclose(kc[l, slot[r]].reshape(-1), want, atol=1e-12)
            # head split: output o goes to head o // Dh, dim o % Dh
            assert np.allclose(kc[l, slot[r], 1, 0], want[Dh], atol=1e-12)
    untouched = [s for s in range(10) if s not in (5, 3, 0)]
    assert np.all(np.isnan(kc[:, untouched]))


# -------------------------------------------------------------- P6 router

def test_p6_router_zero_weights_tie():
    rng = np.random.default_rng(9)
    h = rng.standard_normal((10, 16))
    cos, prob, mask, all_exit = O.route(h, h, None, 1e-6, np.zeros((4, 16)), np.ones(4),
                                         -np.inf, 0.5)
    assert np.all(prob == 0.5)           # SiLU(0) = 0, sigmoid(0) = 1/2
    assert np.all(mask == 0) and all_exit == 0   # strict: a tie continues


def test_p6_router_param_count():
    g = _gold("tide_router_params.json")
    d, b = g["d"], g["b"]
    n_params = np.zeros((b, d)).size + np.zeros((1, b)).size
    assert n_params == 524_416
    assert round(n_params / 1000) == g["approx_params_thousands"]


def test_p6_router_matches_torch_functional():
    import torch.nn.functional as F
    rng = np.random.default_rng(10)
    n, d, b = 37, 24, 6
    hp = rng.standard_normal((n, d))
    hc = rng.standard_normal((n, d)) * rng.uniform(0.1, 5, (n, 1))
    gam = rng.uniform(0.5, 1.5, d)
    wd = rng.standard_normal((b, d)) / math.sqrt(d)
    wu = rng.standard_normal(b)
    eps = 1e-5
    _, prob, _, _ = O.route(hp, hc, gam, eps, wd, wu, -np.inf, -np.inf)
    t = torch.from_numpy(hc)
    x = F.rms_norm(t, (d,), weight=torch.from_numpy(gam), eps=eps)
    z = F.linear(F.silu(F.linear(x, torch.from_numpy(wd))), torch.from_numpy(wu)[None])
    ref = torch.sigmoid(z)[:, 0].numpy()
    assert np.allclose(prob, ref, atol=1e-14, rtol=0)


# ------------------------------------------------------------- P7 RMSNorm

def test_p7_rmsnorm_scale_invariance():
    rng = np.random.default_rng(11)
    h = rng.standard_normal((20, 32))
    wd = rng.standard_normal((8, 32))
    wu = rng.standard_normal(8)
    _, p1, _, _ = O.route(h, h, None, 0.0, wd, wu, -np.inf, -np.inf)
    for c in (1e-3, 0.5, 7.0, 1e4):
        _, pc, _, _ = O.route(h, c * h, None, 0.0, wd, wu, -np.inf, -np.inf)
        assert np.allclose(p1, pc, atol=1e-13, rtol=0)
    # eps matters only at small scale: p(c h) -> p(0) = sigmoid(W_up . SiLU(0))
    _, p0, _, _ = O.route(h, 1e-9 * h, None, 1e-2, wd, wu, -np.inf, -np.inf)
    assert np.allclose(p0, 0.5, atol=1e-6)


# ------------------------------------------------------------- P8 dequant

def test_p8_dequant_hand_example():
    g = _gold("w4_dequant_hand.json")
    got = O.dequant_w4(np.array(g["q_bytes"], np.uint8), np.array(g["scale"]),
                       np.array(g["zero"]), g["group"])
    assert np.array_equal(got, np.array(g["expected"]))


@pytest.mark.parametrize("group,sz", [(32, "f32"), (64, "bf16"), (128, "bf16")])
def test_p8_round_to_nearest_error_bound(group, sz):
    from synth.generate import quantize_w4
    g = torch.Generator().manual_seed(group)
    w = torch.randn((16, 512), generator=g) / 20
    q, s, z = quantize_w4(w, group, sz)
    deq = O.dequant_w4(q.numpy(), s.float().numpy(), z.float().numpy(), group)
    sf = np.repeat(s.float().numpy().astype(np.float64), group, axis=-1)
    err = np.abs(deq - w.numpy().astype(np.float64))
    assert np.all(err <= sf * (0.5 + 1e-5))


# ------------------------------------------------------ P9 KV integrity

def test_p9_kv_integrity_full_schedule():
    """Every (token, layer > e) slot is written exactly once and nothing
    else changes (River-LLM, 研究动机: Intrinsic KV Integrity)."""
    rng = np.random.default_rng(12)
    L, d, Hkv, Dh, n, n_slots = 8, 16, 2, 4, 24, 40
    slot = rng.permutation(n_slots)[:n]
    exits = rng.choice([2, 4, 6, 8], size=n)
    wk = _hand_w4(L, Hkv * Dh, d, 8, rng)
    wv = _hand_w4(L, Hkv * Dh, d, 8, rng)
    h = rng.standard_normal((n, d))
    kc = np.full((L, n_slots, Hkv, Dh), np.nan)
    vc = kc.copy()
    written = {}
    for e in (2, 4, 6, 8):
        rows = np.flatnonzero(exits == e)
        if e == L or len(rows) == 0:
            continue
        sub = lambda w: {"q": w["q"][e:], "scale": w["scale"][e:], "zero": w["zero"][e:], "group": 8}
        k2, v2 = O.kv_fill(h, rows, len(rows), slot, None, sub(wk), sub(wv), Hkv, Dh,
                           kc[e:], vc[e:])
        for l in range(L - e):
            for r in rows:
                key = (e + l, int(slot[r]))
                written[key] = written.get(key, 0) + 1
        kc[e:], vc[e:] = k2, v2
    assert all(c == 1 for c in written.values())
    expect = {(l, int(slot[r])) for r in range(n) for l in range(exits[r], L)}
    assert set(written) == expect
    for l in range(L):
        for s in range(n_slots):
            filled = not np.any(np.isnan(kc[l, s]))
            assert filled == ((l, s) in expect)
            assert filled == (not np.any(np.isnan(vc[l, s])))


# ----------------------------------------------------------- P10 batch rule

def test_p10_batch_rule_is_min_rule():
    rng = np.random.default_rng(13)
    d = 12
    wd = rng.standard_normal((4, d)); wu = rng.standard_normal(4)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        hp = rng.standard_normal((n, d))
        hc = hp + rng.uniform(0, 1.5) * rng.standard_normal((n, d))
        tau = float(rng.uniform(-0.5, 1.0)); theta = float(rng.uniform(0, 1))
        cos, prob, mtok, all_tok = O.route(hp, hc, None, 1e-6, wd, wu, tau, theta, O.RULE_TOKEN)
        _, _, mb, all_b = O.route(hp, hc, None, 1e-6, wd, wu, tau, theta, O.RULE_BATCH_MIN)
        want = int(cos.min() > tau and prob.min() > theta)
        assert all_tok == all_b == want
        assert np.all(mb == want)
        assert all_tok == int(np.all(mtok == 1))
    # adversarial: one token exactly at the threshold holds the batch back
    hp = rng.standard_normal((4, d)); hc = hp.copy()
    _, _, m, a = O.route(hp, hc, None, 1e-6, None, None, 1.0, -np.inf, O.RULE_BATCH_MIN)
    assert a == 0 and np.all(m == 0)     # cos == 1 == tau is not > tau
    _, _, m, a = O.route(hp, hc, None, 1e-6, wd, wu, 1.0, -np.inf, O.RULE_TOKEN)
    assert a == 0 and np.all(m == 0)     # the same with the router on
    _, _, m, a = O.route(hp, hc, None, 1e-6, 0 * wd, wu, -np.inf, 0.5, O.RULE_TOKEN)
    assert a == 0 and np.all(m == 0)     # prob == 0.5 == theta is not > theta
    _, _, m, a = O.route(hp[:0], hc[:0], None, 1e-6, None, None, 0.0, 0.0)
    assert a == 0 and m.size == 0


# --------------------------------------------------- P11 generator shape

def test_p11_cosine_rises_with_depth():
    from synth import get_config
    from synth.generate import hidden_states
    for idx in (0, 1):
        cfg = get_config(idx)
        hs = hidden_states(cfg, 256, range(0, cfg.L + 1))
        means = []
        for l in range(1, cfg.L + 1):
            c, *_ = O.route(hs[l - 1].double().numpy(), hs[l].double().numpy(), None,
                            1e-6, None, None, -np.inf, -np.inf)
            means.append(c.mean())
        assert all(b > a for a, b in zip(means, means[1:]))


# ------------------------------------------------- P12 exit projection

def test_p12_exit_projection_closed_forms():
    """RMSNorm by hand: [3, 4] has mean square 12.5."""
    z = np.zeros((1, 2))
    o = O.exit_projection(np.array([[3.0, 4.0]]), None, 1, None, 0.0, z)
    assert np.allclose(o[0], [3 * math.sqrt(2) / 5, 4 * math.sqrt(2) / 5], atol=1e-15, rtol=0)
    # eps adds to the mean square: 12.5 + 12.5 = 25
    o = O.exit_projection(np.array([[3.0, 4.0]]), None, 1, None, 12.5, z)
    assert np.allclose(o[0], [0.6, 0.8], atol=1e-15, rtol=0)
    # one feature: 3 / sqrt(9 + 16)
    o = O.exit_projection(np.array([[3.0]]), None, 1, np.array([2.0]), 16.0, np.zeros((1, 1)))
    assert np.allclose(o[0], [1.2], atol=1e-15, rtol=0)
    # a constant row normalizes to gamma (times its sign)
    g = np.linspace(-2, 3, 16)
    for c in (-5.0, 0.25, 40.0):
        o = O.exit_projection(np.full((1, 16), c), None, 1, g, 0.0, np.zeros((1, 16)))
        assert np.allclose(o[0], np.sign(c) * g, atol=1e-14, rtol=0)


def test_p12_exit_projection_unit_rms_and_scale():
    rng = np.random.default_rng(12)
    h = rng.standard_normal((9, 48)) * rng.uniform(0.01, 100, (9, 1))
    z = np.zeros_like(h)
    o = O.exit_projection(h, None, 9, None, 0.0, z)
    assert np.allclose(np.mean(o * o, axis=1), 1.0, atol=1e-13, rtol=0)
    for c in (1e-3, 3.0, 1e5):
        assert np.allclose(O.exit_projection(c * h, None, 9, None, 0.0, z), o, atol=1e-13, rtol=0)
    assert np.allclose(O.exit_projection(-h, None, 9, None, 0.0, z), -o, atol=1e-15, rtol=0)
    # a zero row with eps = 0 is 0/0
    o0 = O.exit_projection(np.zeros((1, 8)), None, 1, None, 0.0, np.zeros((1, 8)))
    assert np.isnan(o0).all()


def test_p12_exit_projection_matches_torch_rms_norm():
    import torch.nn.functional as F
    rng = np.random.default_rng(13)
    h = rng.standard_normal((30, 64))
    g = rng.standard_normal(64)
    eps = 1e-2
    o = O.exit_projection(h, None, 30, g, eps, np.zeros_like(h))
    ref = F.rms_norm(torch.from_numpy(h), (64,), weight=torch.from_numpy(g), eps=eps).numpy()
    assert np.allclose(o, ref, atol=1e-14, rtol=0)


def test_p12_exit_projection_scatter():
    """Rows land at row_ids[r]; everything else keeps its old value."""
    import torch.nn.functional as F
    rng = np.random.default_rng(14)
    n, d, n_out = 40, 16, 64
    h = rng.standard_normal((n, d))
    g = rng.standard_normal(d)
    mask = (rng.random(n) < 0.4).astype(np.uint8)
    row_ids = rng.permutation(n_out)[:n]
    c = O.compact(mask, h, row_ids)
    sentinel = np.full((n_out, d), np.nan)
    o = O.exit_projection(h, c["exit_idx"], c["counts"][1], g, 1e-6, sentinel, row_ids)
    normed = F.rms_norm(torch.from_numpy(h), (d,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    ext = set(c["exit_idx"].tolist())
    for r in range(n):
        if r in ext:
            assert np.allclose(o[row_ids[r]], normed[r], atol=1e-14, rtol=0)
    touched = {int(row_ids[r]) for r in ext}
    for q in range(n_out):
        if q not in touched:
            assert np.isnan(o[q]).all()
    # m counts rows of row_idx; out-of-range rows and destinations are skipped
    idx = np.array([3, -1, n + 5, 7, 9])
    ids = np.arange(n)
    ids[7] = n_out + 1
    o = O.exit_projection(h, idx, 4, None, 0.0, np.full((n_out, d), np.nan), ids)
    plain = F.rms_norm(torch.from_numpy(h[3]), (d,), eps=0.0).numpy()
    assert np.allclose(o[3], plain, atol=1e-14, rtol=0)
    assert np.isnan(np.delete(o, 3, axis=0)).all()


# ------------------------------------------- P13 real-layer fill and RoPE

def _rope_tables(n_pos, hd, base):
    """cos / sin of p * base^(-2i/hd), the standard rotary frequencies."""
    inv = base ** (-np.arange(0, hd, 2) / hd)
    ang = np.arange(n_pos)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def test_p13_rope_is_complex_rotation():
    """Pair (x_i, x_{i+hd/2}) as the complex number x_i + j x_{i+hd/2},
    turned by e^{j angle}."""
    rng = np.random.default_rng(21)
    hd = 16
    x = rng.standard_normal((5, 3, hd))
    ang = rng.uniform(-7, 7, (5, 1, hd // 2))
    y = O.rope_half(x, np.cos(ang), np.sin(ang))
    z = (x[..., : hd // 2] + 1j * x[..., hd // 2:]) * np.exp(1j * ang)
    assert np.allclose(y[..., : hd // 2], z.real, atol=1e-14, rtol=0)
    assert np.allclose(y[..., hd // 2:], z.imag, atol=1e-14, rtol=0)


def test_p13_rope_relative_position():
    rng = np.random.default_rng(22)
    hd = 64
    cos, sin = _rope_tables(300, hd, 10000.0)
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    rq = lambda v, p: O.rope_half(v, cos[p], sin[p])
    for p1, p2, sh in ((3, 10, 100), (50, 7, 33), (0, 0, 250)):
        a = rq(q, p1) @ rq(k, p2)
        b = rq(q, p1 + sh) @ rq(k, p2 + sh)
        assert abs(a - b) <= 1e-10 * (abs(a) + 1)
    assert np.allclose(rq(q, 0), q, atol=0, rtol=0)                      # position 0
    assert np.allclose(np.linalg.norm(rq(q, 123)), np.linalg.norm(q), atol=1e-12, rtol=0)


def _layer_case(rng, n_layers=2, d=64, hkv=2, hd=16, group=16, n=7):
    W = rng.standard_normal((2, n_layers, hkv * hd, d)) / math.sqrt(d)
    ws = []
    for which in range(2):
        q, sc, zp = [], [], []
        for l in range(n_layers):
            qq, ss, zz = _quant_np(W[which, l], group)
            q.append(qq)
            sc.append(ss)
            zp.append(zz)
        ws.append({"q": np.stack(q), "scale": np.stack(sc), "zero": np.stack(zp), "group": group})
    h = rng.standard_normal((n, d))
    return h, ws[0], ws[1]


def _quant_np(w, group):
    """Round-to-nearest int4 of one [n_out][d] matrix (test data only)."""
    n_out, d = w.shape
    g = w.reshape(n_out, d // group, group)
    lo, hi = g.min(-1), g.max(-1)
    sc = np.where(hi > lo, (hi - lo) / 15, 1.0)
    zp = -lo / sc
    qv = np.clip(np.rint(g / sc[..., None] + zp[..., None]), 0, 15).astype(np.uint8).reshape(n_out, d)
    return (qv[:, 0::2] | (qv[:, 1::2] << 4)).astype(np.uint8), sc, zp


def test_p13_layer_fill_without_extras_is_linear_fill():
    rng = np.random.default_rng(23)
    h, wk, wv = _layer_case(rng)
    maps = rng.standard_normal((2, 64, 64)) / 8
    rows = np.array([4, 0, 6])
    K0, V0 = O.kv_fill_rows(h, rows, 3, maps, wk, wv)
    K1, V1 = O.kv_fill_layer_rows(h, rows, 3, maps, wk, wv)
    assert np.array_equal(K0, K1) and np.array_equal(V0, V1)


def test_p13_layer_fill_matches_torch():
    """Input RMSNorm, biases and RoPE on K, rebuilt from torch.nn.functional
    and torch complex arithmetic in float64."""
    import torch.nn.functional as F
    rng = np.random.default_rng(24)
    nl, d, hkv, hd = 2, 64, 2, 16
    h, wk, wv = _layer_case(rng, nl, d, hkv, hd)
    maps = np.eye(d)[None] + rng.standard_normal((nl, d, d)) / 20
    gamma = 1 + 0.1 * rng.standard_normal((nl, d))
    bk = rng.standard_normal((nl, hkv * hd))
    bv = rng.standard_normal((nl, hkv * hd))
    cos, sin = _rope_tables(40, hd, 500000.0)
    pos = rng.permutation(40)[: h.shape[0]]
    rows = np.array([6, 2, 3, 0])
    eps = 1e-5
    K, V = O.kv_fill_layer_rows(h, rows, 4, maps, wk, wv, gamma, eps, bk, bv, pos, cos, sin, hkv, hd)
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    ang = T(np.arctan2(sin, cos))
    for l in range(nl):
        x = T(h[rows]) @ T(maps[l]).T
        xn = F.rms_norm(x, (d,), weight=T(gamma[l]), eps=eps)
        Wk = T(O.dequant_w4(wk["q"][l], wk["scale"][l], wk["zero"][l], wk["group"]))
        Wv = T(O.dequant_w4(wv["q"][l], wv["scale"][l], wv["zero"][l], wv["group"]))
        k = F.linear(xn, Wk, T(bk[l])).reshape(len(rows), hkv, hd)
        v = F.linear(xn, Wv, T(bv[l]))
        zc = torch.complex(k[..., : hd // 2], k[..., hd // 2:])
        rot = torch.polar(torch.ones_like(ang), ang)[torch.from_numpy(pos[rows])][:, None, :]
        zr = zc * rot
        kr = torch.cat([zr.real, zr.imag], dim=-1).reshape(len(rows), hkv * hd)
        assert np.allclose(K[l], kr.numpy(), atol=1e-12, rtol=0)
        assert np.allclose(V[l], v.numpy(), atol=1e-12, rtol=0)


def test_p13_layer_fill_norm_scale_invariance_and_bias():
    rng = np.random.default_rng(25)
    nl, d, hkv, hd = 2, 64, 2, 16
    h, wk, wv = _layer_case(rng, nl, d, hkv, hd)
    gamma = 1 + 0.1 * rng.standard_normal((nl, d))
    K1, V1 = O.kv_fill_layer_rows(h, None, 5, None, wk, wv, gamma, 0.0)
    K2, V2 = O.kv_fill_layer_rows(37.0 * h, None, 5, None, wk, wv, gamma, 0.0)
    assert np.allclose(K1, K2, atol=1e-12, rtol=0) and np.allclose(V1, V2, atol=1e-12, rtol=0)
    # zero weights (q equal to the zero point): K is the rotated bias, V the bias
    wz = {"q": np.full_like(wk["q"], 0x33), "scale": np.ones_like(wk["scale"]),
          "zero": np.full_like(wk["zero"], 3.0), "group": wk["group"]}
    bk = rng.standard_normal((nl, hkv * hd))
    bv = rng.standard_normal((nl, hkv * hd))
    cos, sin = _rope_tables(10, hd, 10000.0)
    pos = np.arange(h.shape[0]) + 2
    K, V = O.kv_fill_layer_rows(h, None, 5, None, wz, wz, gamma, 1e-6, bk, bv, pos, cos, sin, hkv, hd)
    for l in range(nl):
        assert np.array_equal(V[l], np.broadcast_to(bv[l], V[l].shape))
        for t in range(5):
            ang = np.arctan2(sin[pos[t]], cos[pos[t]])
            b = bk[l].reshape(hkv, hd)
            z = (b[:, : hd // 2] + 1j * b[:, hd // 2:]) * np.exp(1j * ang)
            assert np.allclose(K[l, t], np.concatenate([z.real, z.imag], axis=1).ravel(),
                               atol=1e-13, rtol=0)


# ------------------------------------------------------- P14 decode step

def _decode_case(rng, rule=O.RULE_TOKEN, router=False):
    L, d, Hkv, Dh, n, n_slots = 8, 16, 2, 4, 20, 32
    slot = rng.permutation(n_slots)[:n]
    wk = _hand_w4(L, Hkv * Dh, d, 8, rng)
    wv = _hand_w4(L, Hkv * Dh, d, 8, rng)
    hs = [rng.standard_normal((n, d))]
    for l in range(1, L + 1):
        hs.append(hs[-1] + rng.uniform(0.1, 1.2, (n, 1)) * rng.standard_normal((n, d)))
    cks = []
    for e in (2, 3, 5, 6):
        c = {"layer": e, "h_prev": hs[e - 1], "h_cur": hs[e], "tau": 0.55, "theta": -np.inf,
             "maps": None if e % 2 else np.eye(d)[None] + 0.05 * rng.standard_normal((L - e, d, d))}
        if router:
            c["w_down"] = rng.standard_normal((4, d))
            c["w_up"] = rng.standard_normal(4)
            c["tau"], c["theta"] = 0.93, 0.5
        cks.append(c)
    kc = np.full((L, n_slots, Hkv, Dh), np.nan)
    return cks, L, slot, wk, wv, Hkv, Dh, kc


def test_p14_decode_step_first_passing_checkpoint_and_integrity():
    rng = np.random.default_rng(31)
    cks, L, slot, wk, wv, Hkv, Dh, kc = _decode_case(rng, router=True)
    ex, K, V = O.decode_step(cks, L, O.RULE_TOKEN, slot, wk, wv, Hkv, Dh, kc, kc)
    n = len(ex)
    # each token exits at the first checkpoint its own decision passes
    for i in range(n):
        first = L
        for c in cks:
            cos, prob, _, _ = O.route(c["h_prev"][i:i + 1], c["h_cur"][i:i + 1], None, 1e-6,
                                      c.get("w_down"), c.get("w_up"), c["tau"], c["theta"])
            if cos[0] > c["tau"] and prob[0] > c["theta"]:
                first = c["layer"]
                break
        assert ex[i] == first
    assert 0 < np.sum(ex < L) < n
    # Intrinsic KV integrity: slot s of cache layer j is written iff its
    # token exited before block j + 1; the count matches the schedule's
    filled = ~np.isnan(K).any(axis=(2, 3))
    for j in range(L):
        for i in range(n):
            assert filled[j, slot[i]] == (ex[i] <= j)
    assert filled.sum() == O.exit_schedule_ops(ex, L)["filled"]
    assert np.array_equal(filled, ~np.isnan(V).any(axis=(2, 3)))


def test_p14_decode_step_one_checkpoint_is_route_compact_fill():
    rng = np.random.default_rng(32)
    cks, L, slot, wk, wv, Hkv, Dh, kc = _decode_case(rng)
    c = cks[1]
    ex, K, V = O.decode_step([c], L, O.RULE_TOKEN, slot, wk, wv, Hkv, Dh, kc, kc)
    _, _, m, _ = O.route(c["h_prev"], c["h_cur"], None, 1e-6, None, None, c["tau"], c["theta"])
    rows = O.compact(m, None)["exit_idx"]
    e = c["layer"]
    sub = lambda w: {"q": w["q"][e:], "scale": w["scale"][e:], "zero": w["zero"][e:], "group": 8}
    k2, v2 = O.kv_fill(c["h_cur"], rows, len(rows), slot, c["maps"], sub(wk), sub(wv), Hkv, Dh,
                       kc[e:], kc[e:])
    assert np.array_equal(np.flatnonzero(ex == e), rows)
    assert np.array_equal(K[e:], k2, equal_nan=True) and np.array_equal(V[e:], v2, equal_nan=True)
    assert np.isnan(K[:e]).all()


def test_p14_decode_step_batch_rule():
    """Under the batch rule a checkpoint lets every running token exit or
    none, and it does so exactly when the smallest cosine of the running
    tokens passes (River-LLM step 3)."""
    rng = np.random.default_rng(33)
    cks, L, slot, wk, wv, Hkv, Dh, kc = _decode_case(rng)
    n = cks[0]["h_cur"].shape[0]
    # some but not all tokens pass the first two checkpoints; the third one
    # passes for everybody (a tiny step keeps cos near 1)
    for c in cks:
        c["tau"] = 0.85
    cks[2]["h_cur"] = cks[2]["h_prev"] * 1.0001
    ex, K, _ = O.decode_step(cks, L, O.RULE_BATCH_MIN, slot, wk, wv, Hkv, Dh, kc, kc)
    alive = np.ones(n, bool)
    for c in cks:
        cos, _, _, _ = O.route(c["h_prev"], c["h_cur"], None, 1e-6, None, None, -np.inf, -np.inf)
        passes = alive.any() and cos[alive].min() > c["tau"]
        assert np.array_equal(ex == c["layer"], alive & passes)
        alive &= ~passes
    assert np.all(ex == cks[2]["layer"])


# ------------------------------------------------ P15 router calibration

def _calib_case(rng, n=96, d=24, b=6):
    h = rng.standard_normal((n, d)) * rng.uniform(0.5, 2.0, (n, 1))
    v = rng.standard_normal(d)
    y = ((h @ v) / np.linalg.norm(h, axis=1) > 0.1).astype(np.uint8)     # learnable from h
    W0 = rng.standard_normal((b, d)) / math.sqrt(d)
    w0 = rng.standard_normal(b) / math.sqrt(b)
    return h, y, W0, w0


def test_p15_router_fit_matches_torch_adam():
    """The same model, loss and optimizer built from torch.nn.functional,
    autograd and torch.optim.Adam in float64."""
    import torch.nn.functional as F
    rng = np.random.default_rng(41)
    h, y, W0, w0 = _calib_case(rng)
    n, d = h.shape
    gam = 1 + 0.1 * rng.standard_normal(d)
    orders = np.stack([rng.permutation(n) for _ in range(3)])
    W, w, loss = O.router_fit(h, y, W0, w0, 3, 20, orders, gam, 1e-5, lr=1e-2)
    Wt = torch.tensor(W0, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([Wt, wt], lr=1e-2, betas=(0.9, 0.999), eps=1e-8)
    H = torch.from_numpy(h)
    Y = torch.from_numpy(y.astype(np.float64))
    tl = []
    for e in range(3):
        tot = 0.0
        for s0 in range(0, n, 20):
            rows = torch.from_numpy(orders[e][s0:s0 + 20])
            x = F.rms_norm(H[rows], (d,), weight=torch.from_numpy(gam), eps=1e-5)
            z = F.linear(F.silu(F.linear(x, Wt)), wt[None])[:, 0]
            lb = F.binary_cross_entropy_with_logits(z, Y[rows])
            opt.zero_grad()
            lb.backward()
            opt.step()
            tot += float(lb.detach()) * len(rows)
        tl.append(tot / n)
    assert np.allclose(W, Wt.detach().numpy(), atol=1e-12, rtol=0)
    assert np.allclose(w, wt.detach().numpy(), atol=1e-12, rtol=0)
    assert np.allclose(loss, tl, atol=1e-12, rtol=0)
    assert loss[-1] < loss[0]


def test_p15_router_fit_first_step_is_signed_lr():
    """Adam's first update is -lr g / (|g| + eps): -lr sign(g) wherever the
    gradient is well above eps; the gradient's sign from central finite
    differences of the mean BCE."""
    rng = np.random.default_rng(42)
    h, y, W0, w0 = _calib_case(rng, n=40, d=10, b=3)
    lr = 1e-3
    W1, w1, _ = O.router_fit(h, y, W0, w0, 1, 40, lr=lr)

    def loss(W, w):
        x = h / np.sqrt(np.mean(h * h, axis=1) + 1e-6)[:, None]
        u = x @ W.T
        z = (u / (1 + np.exp(-u))) @ w
        return float(np.mean(np.logaddexp(0, z) - y * z))
    step = 1e-6
    for (i, j) in [(0, 0), (1, 4), (2, 9), (0, 7)]:
        Wp, Wm = W0.copy(), W0.copy()
        Wp[i, j] += step
        Wm[i, j] -= step
        gfd = (loss(Wp, w0) - loss(Wm, w0)) / (2 * step)
        assert abs(gfd) > 1e-5
        assert np.isclose(W1[i, j] - W0[i, j], -lr * np.sign(gfd), rtol=1e-3, atol=0)
    for k in range(3):
        wp, wm = w0.copy(), w0.copy()
        wp[k] += step
        wm[k] -= step
        gfd = (loss(W0, wp) - loss(W0, wm)) / (2 * step)
        assert np.isclose(w1[k] - w0[k], -lr * np.sign(gfd), rtol=1e-3, atol=0)


def test_p15_router_zero_up_projection():
    """With w_up = 0 every probability is 1/2: the first epoch's loss is
    log 2 and W_down gets no gradient in the first step."""
    rng = np.random.default_rng(43)
    h, y, W0, _ = _calib_case(rng, n=30)
    W1, w1, loss = O.router_fit(h, y, W0, np.zeros(6), 1, 30)
    assert abs(loss[0] - math.log(2)) < 1e-15
    assert np.array_equal(W1, W0)
    assert np.all(np.abs(np.abs(w1) - 1e-3) < 1e-9)


def test_p15_router_labels_match_scipy_cosine():
    from scipy.spatial.distance import cosine
    rng = np.random.default_rng(44)
    hk = rng.standard_normal((50, 12))
    hL = hk + rng.uniform(0, 0.5, (50, 1)) * rng.standard_normal((50, 12))
    y = O.router_labels(hk, hL, 0.98)
    ref = np.array([1 - cosine(hk[i], hL[i]) > 0.98 for i in range(50)], dtype=np.uint8)
    assert np.array_equal(y, ref) and 0 < y.sum() < 50


# --------------------------------------------------------- mutation checks

def _mutant_oracle(old, new):
    """A copy of the oracle module with one textual slip planted."""
    import inspect
    import types
    import oracle.river_oracle as R
    src = inspect.getsource(R)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


MUTANTS = [
    # wrong operand in the cosine denominator
    ("cos[ok] = dot[ok] / np.sqrt(na[ok] * nb[ok])",
     "cos[ok] = dot[ok] / np.sqrt(na[ok] * na[ok])", "test_p1_cosine_matches_scipy_and_bounds"),
    # RMSNorm without the mean over d
    ("r = 1.0 / np.sqrt(nb / d + eps)", "r = 1.0 / np.sqrt(nb + eps)",
     "test_p6_router_matches_torch_functional"),
    # gamma dropped
    ("x = b * g[None, :] * r[:, None]", "x = b * r[:, None]",
     "test_p6_router_matches_torch_functional"),
    # SiLU replaced by a sigmoid
    ("act = u * _sigmoid(u)", "act = _sigmoid(u)", "test_p6_router_zero_weights_tie"),
    # non-strict threshold
    ("e = (cos > tau) & (prob > theta)", "e = (cos >= tau) & (prob > theta)",
     "test_p10_batch_rule_is_min_rule"),
    # inverted partition
    ("if mask[i] != 0:", "if mask[i] == 0:", "test_p4_compaction_exhaustive_small"),
    # nibble order swapped
    ("lo = (q & 0x0F).astype(np.float64)", "lo = (q >> 4).astype(np.float64)",
     "test_p8_dequant_hand_example"),
    # zero point applied after the scale
    ("return (vals - z) * s", "return vals * s - z", "test_p8_dequant_hand_example"),
    # map applied transposed
    ("xh = x if maps is None else x @ _f64(maps[l]).T",
     "xh = x if maps is None else x @ _f64(maps[l])", "test_p5_map_orientation_and_slots"),
    # projection weights applied transposed
    ("K[l] = xh @ Wk.T", "K[l] = (xh @ Wk.T)[:, ::-1]", "test_p5_identity_fill_is_direct_projection"),
    # ridge term dropped
    ("G = X.T @ X + lam * np.eye(d_in)", "G = X.T @ X + np.eye(d_in)",
     "test_p3_ridge_matches_lstsq_and_sklearn"),
    # ridge result left input-major
    ("out[t] = W.T", "out[t] = W.reshape(W.shape[::-1])", "test_p3_ridge_closed_forms"),
    # RMSNorm over the sum instead of the mean
    ("ms = np.mean(x * x)", "ms = np.sum(x * x)", "test_p12_exit_projection_closed_forms"),
    # eps dropped from the final norm
    ("np.sqrt(ms + eps)", "np.sqrt(ms)", "test_p12_exit_projection_closed_forms"),
    # gamma dropped from the final norm
    ("o[dst] = g * x / np.sqrt(ms + eps)", "o[dst] = x / np.sqrt(ms + eps)",
     "test_p12_exit_projection_matches_torch_rms_norm"),
    # scatter ignores the row ids
    ("dst = r if row_ids is None else int(row_ids[r])", "dst = r",
     "test_p12_exit_projection_scatter"),
    # rotation with the wrong sign
    ("np.concatenate([a * c - b * s, a * s + b * c]", "np.concatenate([a * c + b * s, a * s + b * c]",
     "test_p13_rope_is_complex_rotation"),
    # interleaved pairs instead of halves
    ("a, b = x[..., :half], x[..., half:]", "a, b = x[..., 0::2], x[..., 1::2]",
     "test_p13_layer_fill_matches_torch"),
    # the layer norm's weight dropped
    ("xh = _f64(gamma[l])[None, :] * xh / np.sqrt(ms + eps)[:, None]",
     "xh = xh / np.sqrt(ms + eps)[:, None]", "test_p13_layer_fill_matches_torch"),
    # every row rotated at position 0
    ("c = _f64(cos)[p][:, None, :]", "c = _f64(cos)[p * 0][:, None, :]",
     "test_p13_layer_fill_matches_torch"),
    # K bias dropped
    ("K[l] += _f64(bk[l])[None, :]", "K[l] += 0.0", "test_p13_layer_fill_norm_scale_invariance_and_bias"),
    # an exited token takes part in later checkpoints again
    ("dec = (m != 0) & alive", "dec = (m != 0)",
     "test_p14_decode_step_first_passing_checkpoint_and_integrity"),
    # the batch rule taking any running token instead of every one
    ("every = alive.any() and bool(np.all(dec[alive]))", "every = bool(np.any(dec[alive]))",
     "test_p14_decode_step_batch_rule"),
    # SiLU's derivative without its second term
    ("gu = gz[:, None] * w[None, :] * (su * (1.0 + u * (1.0 - su)))",
     "gu = gz[:, None] * w[None, :] * su", "test_p15_router_fit_matches_torch_adam"),
    # Adam without bias correction
    ("mh = M / (1.0 - beta1 ** t)", "mh = M", "test_p15_router_fit_first_step_is_signed_lr"),
    # batch loss averaged over the whole set instead of the batch
    ("gz = (p - yy) / B", "gz = (p - yy) / n", "test_p15_router_fit_matches_torch_adam"),
    # label threshold not strict
    ("return (cos > tau_c).astype(np.uint8)", "return (cos >= 0.9).astype(np.uint8)",
     "test_p15_router_labels_match_scipy_cosine"),
    # off-by-one in the filled layers
    ("filled = sum(n_layers - x for x in e)", "filled = sum(n_layers - x + 1 for x in e)",
     "test_p2_tide_figure2_worked_example"),
]


@pytest.mark.parametrize("old,new,pin", MUTANTS, ids=[m[2] + ":" + m[1][:24] for m in MUTANTS])
def test_mutation_is_caught(monkeypatch, old, new, pin):
    mod = _mutant_oracle(old, new)
    for name in O.__all__ if hasattr(O, "__all__") else dir(mod):
        if hasattr(mod, name) and callable(getattr(mod, name)) and hasattr(O, name):
            monkeypatch.setattr(O, name, getattr(mod, name))
    with pytest.raises(AssertionError):
        globals()[pin]()
