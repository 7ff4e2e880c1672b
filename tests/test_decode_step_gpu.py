"""GPU parity of one generation step of the token-level exit loop
(river_decode_step) against the float64 oracle, eagerly and replayed from a
captured HIP graph.

Bars: exit layers bit-exact for tokens whose cosines and probabilities at
every checkpoint they reach lie outside the 1e-4 band around the thresholds
(tokens inside it are excluded and counted; at most an eighth may be); K/V of
filled slots within the fill's bar (per-row relative L2 <= 1e-2); every
other slot keeps its NaN sentinel. A graph replay equals the eager call bit
for bit.
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
from helpers import BAND, KV_TOL, f32, kv_row_errors, np64, w4_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
INF = math.inf


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    tee.river_debug_set_compact_path(0)
    yield


def _kv(cfg, layers):
    w = G.kv_weights(cfg, layers, device="cpu" if cfg.d <= 2048 else DEV)
    return (tuple(t.to(DEV) for t in w["wk"]) + (cfg.group,),
            tuple(t.to(DEV) for t in w["wv"]) + (cfg.group,))


def step_workspace(cfg, n, split=True):
    """split: room for the split reduction of the fills (n <= 64)."""
    d_out = cfg.n_kv_heads * cfg.head_dim if split else 0
    return torch.empty(tee.river_workspace_size(tee.OP_DECODE_STEP, n, cfg.d, d_out, 0, cfg.L),
                       dtype=torch.uint8, device=DEV)


def run_gpu(cks, cfg, wk, wv, slot, rule=O.RULE_TOKEN, caches=None, split=True):
    kc, vc = caches if caches is not None else G.nan_cache(cfg, cfg.L, device=DEV)
    n = cks[0]["h_cur"].shape[0]
    ex = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    ws = step_workspace(cfg, n, split)
    tee.river_decode_step(cks, wk, wv, cfg.n_kv_heads, cfg.head_dim, slot, kc, vc, ex, rule=rule,
                          workspace=ws)
    torch.cuda.synchronize()
    return ex, kc, vc


def oracle_cks(cks):
    out = []
    for c in cks:
        o = {"layer": c["layer"], "h_prev": np64(c["h_prev"]), "h_cur": np64(c["h_cur"]),
             "tau": f32(c["tau"]), "theta": f32(c["theta"])}
        if c.get("w_down") is not None:
            o["w_down"], o["w_up"] = np64(c["w_down"]), np64(c["w_up"])
        out.append(o)
    return out


def band_tokens(cks, ex_ref):
    """Tokens whose cosine or probability at a checkpoint they reached lies
    within the band around the threshold."""
    n = len(ex_ref)
    bad = np.zeros(n, bool)
    for c in oracle_cks(cks):
        cos, prob, _, _ = O.route(c["h_prev"], c["h_cur"], None, 1e-6, c.get("w_down"),
                                  c.get("w_up"), -INF, -INF)
        reach = ex_ref >= c["layer"]
        near = np.abs(cos - c["tau"]) < BAND
        if c.get("w_down") is not None:
            near |= np.abs(prob - c["theta"]) < BAND
        bad |= reach & near
    return bad


def check_step(cfg, cks, ex, kc, vc, slot, wk, wv, rule=O.RULE_TOKEN, sample_per_ck=None):
    """Exit layers against the oracle's; filled slots' K/V against the
    oracle's fill of the GPU's own exits."""
    ocks = oracle_cks(cks)
    n = ex.shape[0]
    # oracle exit layers (no fill: caches of one layer and one slot)
    ex_ref = np.full(n, cfg.L)
    alive = np.ones(n, bool)
    for c in ocks:
        _, _, m, _ = O.route(c["h_prev"], c["h_cur"], None, 1e-6, c.get("w_down"), c.get("w_up"),
                             c["tau"], c["theta"])
        dec = (m != 0) & alive
        if rule == O.RULE_BATCH_MIN:
            dec = alive & (alive.any() and bool(np.all(dec[alive])))
        ex_ref[dec] = c["layer"]
        alive &= ~dec
    bad = band_tokens(cks, ex_ref)
    assert bad.sum() <= max(2, n // 8), f"{bad.sum()} tokens in the threshold band"
    exg = ex.cpu().numpy()
    assert np.array_equal(exg[~bad], ex_ref[~bad])
    # K/V of the filled slots
    slot_np = slot.cpu().numpy()
    for ci, c in enumerate(cks):
        e = c["layer"]
        rows = np.flatnonzero((exg == e) & ~bad)
        if len(rows) == 0:
            continue
        if sample_per_ck is not None and len(rows) > sample_per_ck:
            rows = np.sort(np.random.default_rng(e).choice(rows, sample_per_ck, replace=False))
        maps = c.get("maps")
        K, V = O.kv_fill_rows(np64(c["h_cur"]), rows, len(rows),
                              None if maps is None else maps.float().cpu().numpy(),
                              w4_np(tuple(t[e:] for t in wk[:3]) + (wk[3],)),
                              w4_np(tuple(t[e:] for t in wv[:3]) + (wv[3],)))
        s = torch.from_numpy(slot_np[rows].astype(np.int64)).to(DEV)
        ek = kv_row_errors(kc[e:, s].reshape(cfg.L - e, len(rows), -1), K)
        evv = kv_row_errors(vc[e:, s].reshape(cfg.L - e, len(rows), -1), V)
        assert ek.max() <= KV_TOL and evv.max() <= KV_TOL, (e, ek.max(), evv.max())
    # exactly the slots of cache layers >= exit layer hold values
    nan_k = torch.isnan(kc).all(dim=-1).all(dim=-1).cpu().numpy()       # [L][n_slots]
    nan_v = torch.isnan(vc).all(dim=-1).all(dim=-1).cpu().numpy()
    want = np.ones_like(nan_k)
    for i in range(n):
        want[exg[i]:, slot_np[i]] = False       # the GPU's own exit layers (checked above)
    assert np.array_equal(nan_k, want) and np.array_equal(nan_v, want)
    return exg


def llama1b_checkpoints(cfg, hs):
    """Checkpoints after blocks 8..15, router off, tau_l at the midpoint of
    the two middle oracle cosines of the tokens still running."""
    n = cfg.n_tokens
    alive = np.ones(n, bool)
    cks = []
    for l in cfg.route_layers:
        cos, *_ = O.route(np64(hs[l - 1]), np64(hs[l]), None, 1e-6, None, None, -INF, -INF)
        c = np.sort(cos[alive])
        m = len(c)
        tau = 0.5 * (c[(m - 1) // 2] + c[m // 2]) if m > 1 else (c[0] - 1 if m else 0.0)
        cks.append({"layer": l, "h_prev": hs[l - 1], "h_cur": hs[l], "tau": tau, "theta": -INF})
        alive &= ~(cos > f32(tau))
    return cks


@pytest.mark.parametrize("split", [True, False])
def test_decode_step_llama1b(split):
    """split: the fills' reduction over d runs in parts (64 rows at most)."""
    cfg = get_config(2)
    hs = {l: t.to(DEV) for l, t in G.hidden_states(cfg, cfg.n_tokens, range(7, 17)).items()}
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    cks = llama1b_checkpoints(cfg, hs)
    ex, kc, vc = run_gpu(cks, cfg, wk, wv, slot, split=split)
    exg = check_step(cfg, cks, ex, kc, vc, slot, wk, wv)
    counts = np.bincount(exg, minlength=cfg.L + 1)[8:]
    assert counts[0] >= 28 and counts.sum() == cfg.n_tokens      # about half exit at block 8


@pytest.mark.parametrize("rule", [O.RULE_TOKEN, O.RULE_BATCH_MIN])
def test_decode_step_two_launch_equals_per_checkpoint(rule):
    """Routers off: the two decision launches for all checkpoints and the
    per-checkpoint route/compact launches give the same bits (exit blocks
    and caches)."""
    cfg = get_config(2)
    hs = {l: t.to(DEV) for l, t in G.hidden_states(cfg, cfg.n_tokens, range(7, 17)).items()}
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    cks = llama1b_checkpoints(cfg, hs)
    if rule == O.RULE_BATCH_MIN:
        cos, *_ = O.route(np64(hs[10]), np64(hs[11]), None, 1e-6, None, None, -INF, -INF)
        for c in cks:
            c["tau"] = 2.0
        cks[3]["tau"] = float(cos.min()) - 1e-3
    out = []
    try:
        for path in (0, 1):
            tee.river_debug_set_decode_path(path)
            out.append(run_gpu(cks, cfg, wk, wv, slot, rule=rule))
    finally:
        tee.river_debug_set_decode_path(0)
    (e0, k0, v0), (e1, k1, v1) = out
    assert torch.equal(e0, e1)
    assert torch.equal(k0.view(torch.int16), k1.view(torch.int16))
    assert torch.equal(v0.view(torch.int16), v1.view(torch.int16))
    assert (e0 < cfg.L).any()


def test_decode_step_llama1b_batch_rule():
    """Batch rule: the step lets everybody exit at block 11, where tau
    sits below the smallest cosine, and nobody before."""
    cfg = get_config(2)
    hs = {l: t.to(DEV) for l, t in G.hidden_states(cfg, cfg.n_tokens, range(7, 17)).items()}
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    cks = llama1b_checkpoints(cfg, hs)
    cos, *_ = O.route(np64(hs[10]), np64(hs[11]), None, 1e-6, None, None, -INF, -INF)
    for c in cks:
        c["tau"] = 2.0                           # no token passes (cos <= 1)
    cks[3]["tau"] = float(cos.min()) - 1e-3
    ex, kc, vc = run_gpu(cks, cfg, wk, wv, slot, rule=O.RULE_BATCH_MIN)
    exg = check_step(cfg, cks, ex, kc, vc, slot, wk, wv, rule=O.RULE_BATCH_MIN)
    assert np.all(exg == 11)


def llama8b_checkpoints(cfg, hs):
    """Router checkpoints every four blocks: tau off, theta_11 between the
    13th and 14th largest probabilities, theta_31 = -inf, +inf elsewhere;
    near-identity maps for the fills at 11 and 31."""
    cks = []
    for l in cfg.route_layers:
        wd, wu = (t.to(DEV) for t in G.router_weights(cfg, l))
        c = {"layer": l, "h_prev": hs[l - 1], "h_cur": hs[l], "tau": -INF, "theta": INF,
             "w_down": wd, "w_up": wu}
        if l == 11:
            _, prob, _, _ = O.route(np64(hs[10]), np64(hs[11]), None, 1e-6, np64(wd), np64(wu),
                                    -INF, -INF)
            p = np.sort(prob)[::-1]
            c["theta"] = 0.5 * (p[12] + p[13])
            c["maps"] = G.near_identity_maps(cfg, cfg.L - l, device=DEV)
        if l == 31:
            c["theta"] = -INF
            c["maps"] = G.near_identity_maps(cfg, cfg.L - l, tag="maps31", device=DEV)
        cks.append(c)
    return cks


def test_decode_step_8b_two_launch_equals_per_checkpoint():
    """Routers on at every checkpoint: one route launch for all checkpoints
    plus the decision workgroup give the same bits as the per-checkpoint
    route and compact launches."""
    cfg = get_config("3D")
    n = cfg.n_tokens
    layers = list(cfg.route_layers)
    need = sorted({l - 1 for l in layers} | set(layers))
    hs = G.hidden_states(cfg, n, need, device=DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    cks = llama8b_checkpoints(cfg, hs)
    out = []
    try:
        for path in (0, 1):
            tee.river_debug_set_decode_path(path)
            out.append(run_gpu(cks, cfg, wk, wv, slot))
    finally:
        tee.river_debug_set_decode_path(0)
    (e0, k0, v0), (e1, k1, v1) = out
    assert torch.equal(e0, e1)
    assert torch.equal(k0.view(torch.int16), k1.view(torch.int16))
    assert torch.equal(v0.view(torch.int16), v1.view(torch.int16))
    assert np.sum(e0.cpu().numpy() == 11) == 13


@pytest.mark.parametrize("folded", [False, True])
def test_decode_step_8b_router_and_maps(folded):
    """Llama-3-8B-shape decode (256 tokens, d = 4096, checkpoints every four
    blocks with a router each): tau off, theta_11 between the 13th and 14th
    largest probabilities, theta_31 = -inf, +inf elsewhere; near-identity
    maps for the fills."""
    cfg = get_config("3D")
    n = cfg.n_tokens
    layers = list(cfg.route_layers)
    need = sorted({l - 1 for l in layers} | set(layers))
    hs = G.hidden_states(cfg, n, need, device=DEV)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    cks = []
    for l in layers:
        wd, wu = (t.to(DEV) for t in G.router_weights(cfg, l))
        c = {"layer": l, "h_prev": hs[l - 1], "h_cur": hs[l], "tau": -INF, "theta": INF,
             "w_down": wd, "w_up": wu}
        if l == 11:
            _, prob, _, _ = O.route(np64(hs[10]), np64(hs[11]), None, 1e-6, np64(wd), np64(wu),
                                    -INF, -INF)
            p = np.sort(prob)[::-1]
            c["theta"] = 0.5 * (p[12] + p[13])
            c["maps"] = G.near_identity_maps(cfg, cfg.L - l, device=DEV)
        if l == 31:
            c["theta"] = -INF
            c["maps"] = G.near_identity_maps(cfg, cfg.L - l, tag="maps31", device=DEV)
        cks.append(c)
    if folded:
        # the checkpoints with maps fill through deq([Wk; Wv]) M (river_kv_fold)
        B.fold_checkpoints(cfg, cks, wk, wv, DEV)
    ex, kc, vc = run_gpu(cks, cfg, wk, wv, slot)
    exg = check_step(cfg, cks, ex, kc, vc, slot, wk, wv, sample_per_ck=12)
    assert np.sum(exg == 11) == 13 and np.sum(exg == 31) == n - 13


@pytest.mark.parametrize("case", ["ragged-37", "200-split", "300-no-split", "router-off-maps",
                                  "fp32-tiny", "mixed-routers", "routers-maps"])
def test_decode_step_paths_and_shapes(case):
    """Shapes around the step's paths, each against the oracle and against
    the per-checkpoint launches: 37 tokens (single fill, split reduction,
    ragged tiles), 200 tokens (the split over 64-row tiles, in parts that
    differ between the paths), 300 tokens (no split), maps at two
    router-off checkpoints (two decision launches, a fill per checkpoint),
    fp32 states (the generic fill), and routers at some checkpoints only
    (per-checkpoint launches), and routers at every checkpoint with maps at
    two (the single fill of the others beside a fill per checkpoint with
    maps; the paths split the projection differently). Exit layers agree
    bit for bit; so do the caches wherever both paths fill with the same
    launches."""
    bitwise = case not in ("ragged-37", "200-split", "routers-maps")
    if case == "ragged-37":
        cfg = get_config(2, n_tokens=37)
    elif case == "200-split":
        cfg = get_config(2, n_tokens=200)
    elif case == "300-no-split":
        cfg = get_config(2, n_tokens=300)
    elif case == "router-off-maps":
        cfg = get_config(2)
    elif case == "fp32-tiny":
        cfg = get_config(0)
    else:
        cfg = get_config("3D", n_tokens=64)
    layers = list(cfg.route_layers)
    need = sorted({l - 1 for l in layers} | set(layers))
    hs = {l: t.to(DEV) for l, t in G.hidden_states(cfg, cfg.n_tokens, need).items()}
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    cks = llama1b_checkpoints(cfg, hs)
    if case == "fp32-tiny":
        # cosines a few 1e-5 apart: tau at the middle of the widest gap among
        # the running tokens keeps them out of the band
        alive = np.ones(cfg.n_tokens, bool)
        for c in cks:
            cos, *_ = O.route(np64(c["h_prev"]), np64(c["h_cur"]), None, 1e-6, None, None, -INF, -INF)
            v = np.sort(cos[alive])
            if len(v) < 4:
                c["tau"] = 2.0                 # nobody left to split
                continue
            lo, hi = len(v) // 4, len(v) - len(v) // 4      # keep tokens on both sides
            g = lo + int(np.argmax(np.diff(v)[lo:hi]))
            # no gap twice the band wide: nobody exits here
            c["tau"] = 0.5 * (v[g] + v[g + 1]) if v[g + 1] - v[g] > 2.5 * BAND else 2.0
            alive &= ~(cos > f32(c["tau"]))
    if case == "router-off-maps":
        for c in cks:
            if c["layer"] in (8, 12):
                c["maps"] = G.near_identity_maps(cfg, cfg.L - c["layer"], tag=f"m{c['layer']}").to(DEV)
    if case == "routers-maps":
        # a router at every checkpoint, theta at the middle of the widest gap
        # of the running tokens' probabilities (nobody exits where there is
        # no clear gap); maps for the fills at the second and fifth
        alive = np.ones(cfg.n_tokens, bool)
        for k, c in enumerate(cks):
            wd, wu = (t.to(DEV) for t in G.router_weights(cfg, c["layer"]))
            c["w_down"], c["w_up"], c["tau"], c["theta"] = wd, wu, -INF, INF
            _, prob, _, _ = O.route(np64(c["h_prev"]), np64(c["h_cur"]), None, 1e-6, np64(wd), np64(wu),
                                    -INF, -INF)
            v = np.sort(prob[alive])
            if len(v) >= 8:
                lo, hi = len(v) // 2, len(v) - len(v) // 8
                g = lo + int(np.argmax(np.diff(v)[lo:hi]))
                if v[g + 1] - v[g] > 2.5 * BAND:
                    c["theta"] = 0.5 * (v[g] + v[g + 1])
            alive &= ~(prob > f32(c["theta"]))
            if k in (1, 4):
                c["maps"] = G.near_identity_maps(cfg, cfg.L - c["layer"], tag=f"rm{k}").to(DEV)
    if case == "mixed-routers":
        # the 8B shape's cosines differ in the 8th digit: routers at every
        # other checkpoint decide (tau off, theta at the middle of the widest
        # gap of the running tokens' probabilities); nobody exits elsewhere
        alive = np.ones(cfg.n_tokens, bool)
        for k, c in enumerate(cks):
            c["tau"] = 2.0
            if k % 2:
                continue
            wd, wu = (t.to(DEV) for t in G.router_weights(cfg, c["layer"]))
            c["w_down"], c["w_up"], c["tau"] = wd, wu, -INF
            _, prob, _, _ = O.route(np64(c["h_prev"]), np64(c["h_cur"]), None, 1e-6, np64(wd), np64(wu),
                                    -INF, -INF)
            v = np.sort(prob[alive])
            c["theta"] = INF
            if len(v) >= 4:
                lo, hi = len(v) // 4, len(v) - len(v) // 4
                g = lo + int(np.argmax(np.diff(v)[lo:hi]))
                if v[g + 1] - v[g] > 2.5 * BAND:
                    c["theta"] = 0.5 * (v[g] + v[g + 1])
            alive &= ~(prob > f32(c["theta"]))
    out = []
    try:
        for path in (0, 1):
            tee.river_debug_set_decode_path(path)
            out.append(run_gpu(cks, cfg, wk, wv, slot))
    finally:
        tee.river_debug_set_decode_path(0)
    (e0, k0, v0), (e1, k1, v1) = out
    assert torch.equal(e0, e1)
    if bitwise:
        iv = torch.int16 if k0.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(k0.view(iv), k1.view(iv)) and torch.equal(v0.view(iv), v1.view(iv))
    exg = check_step(cfg, cks, e0, k0, v0, slot, wk, wv)
    assert (exg < cfg.L).any()
    if case == "routers-maps":
        # exits both at checkpoints with maps and at checkpoints without
        got = set(np.unique(np.asarray(exg)[np.asarray(exg) < cfg.L]).tolist())
        with_maps = {cks[1]["layer"], cks[4]["layer"]}
        assert got & with_maps and got - with_maps, got


def test_decode_step_graph_replay():
    """The step captured once into a graph and replayed for three steps with
    new states copied into the captured buffers; each replay equals an eager
    call on the same states, with eager work between the replays."""
    cfg = get_config(2)
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    steps = []
    for k in range(3):
        hs = G.hidden_states(cfg, cfg.n_tokens, range(7, 17), tag=f"step{k}")
        steps.append({l: t.to(DEV) for l, t in hs.items()})
    buf = {l: torch.empty_like(t) for l, t in steps[0].items()}
    cks = llama1b_checkpoints(cfg, steps[0])
    gcks = [dict(c, h_prev=buf[c["layer"] - 1], h_cur=buf[c["layer"]]) for c in cks]
    n = cfg.n_tokens
    kc, vc = G.nan_cache(cfg, cfg.L, device=DEV)
    ex = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    ws = step_workspace(cfg, n)
    for l in buf:
        buf[l].copy_(steps[0][l])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm-up outside the capture
        tee.river_decode_step(gcks, wk, wv, cfg.n_kv_heads, cfg.head_dim, slot, kc, vc, ex,
                              workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        tee.river_decode_step(gcks, wk, wv, cfg.n_kv_heads, cfg.head_dim, slot, kc, vc, ex,
                              workspace=ws)
    for k in range(3):
        for l in buf:
            buf[l].copy_(steps[k][l])
        kc.fill_(float("nan"))
        vc.fill_(float("nan"))
        ex.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        kr, vr, er = kc.clone(), vc.clone(), ex.clone()
        # eager call on the same states, fresh outputs
        eck = [dict(c, h_prev=steps[k][c["layer"] - 1], h_cur=steps[k][c["layer"]]) for c in cks]
        e2, k2, v2 = run_gpu(eck, cfg, wk, wv, slot)
        assert torch.equal(er, e2)
        assert torch.equal(kr.view(torch.int16), k2.view(torch.int16))
        assert torch.equal(vr.view(torch.int16), v2.view(torch.int16))
        assert (er < cfg.L).any()


def test_decode_step_graph_replay_routers_and_maps():
    """Routers at every checkpoint of the Llama-3-8B shape (64 tokens) and
    maps at two: the route launch for all checkpoints, the decision
    workgroup, the single fill of the six without maps and the fills of the
    two with maps, captured once and replayed for three steps with new
    states; each replay equals an eager call bit for bit."""
    cfg = get_config("3D", n_tokens=64)
    n = cfg.n_tokens
    slot = G.slots(cfg, device=DEV)
    wk, wv = _kv(cfg, list(range(1, cfg.L + 1)))
    layers = list(cfg.route_layers)
    need = sorted({l - 1 for l in layers} | set(layers))
    steps = []
    for k in range(3):
        hs = G.hidden_states(cfg, n, need, tag=f"gstep{k}")
        steps.append({l: t.to(DEV) for l, t in hs.items()})
    buf = {l: torch.empty_like(t) for l, t in steps[0].items()}
    cks = []
    for k, l in enumerate(layers):
        wd, wu = (t.to(DEV) for t in G.router_weights(cfg, l))
        c = {"layer": l, "tau": -INF, "theta": INF, "w_down": wd, "w_up": wu}
        # theta between the 8th and 9th largest probabilities of step 0
        _, prob, _, _ = O.route(np64(steps[0][l - 1]), np64(steps[0][l]), None, 1e-6, np64(wd),
                                np64(wu), -INF, -INF)
        p = np.sort(prob)[::-1]
        c["theta"] = 0.5 * (p[7] + p[8])
        if k in (1, 4):
            c["maps"] = G.near_identity_maps(cfg, cfg.L - l, tag=f"gm{k}").to(DEV)
        cks.append(c)
    gcks = [dict(c, h_prev=buf[c["layer"] - 1], h_cur=buf[c["layer"]]) for c in cks]
    kc, vc = G.nan_cache(cfg, cfg.L, device=DEV)
    ex = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    ws = step_workspace(cfg, n)
    for l in buf:
        buf[l].copy_(steps[0][l])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm-up outside the capture
        tee.river_decode_step(gcks, wk, wv, cfg.n_kv_heads, cfg.head_dim, slot, kc, vc, ex,
                              workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        tee.river_decode_step(gcks, wk, wv, cfg.n_kv_heads, cfg.head_dim, slot, kc, vc, ex,
                              workspace=ws)
    for k in range(3):
        for l in buf:
            buf[l].copy_(steps[k][l])
        kc.fill_(float("nan"))
        vc.fill_(float("nan"))
        ex.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        kr, vr, er = kc.clone(), vc.clone(), ex.clone()
        eck = [dict(c, h_prev=steps[k][c["layer"] - 1], h_cur=steps[k][c["layer"]]) for c in cks]
        e2, k2, v2 = run_gpu(eck, cfg, wk, wv, slot)
        assert torch.equal(er, e2)
        assert torch.equal(kr.view(torch.int16), k2.view(torch.int16))
        assert torch.equal(vr.view(torch.int16), v2.view(torch.int16))
        ev = er.cpu().numpy()
        assert (ev < cfg.L).any()
        del kr, vr, e2, k2, v2
