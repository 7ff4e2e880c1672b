"""Benchmark of the per-token exit-and-KV-fill step on one MI355X.

One step is one pass of the whole hot path over one batch: river_route at
the exit layer, river_compact, then river_kv_fill of every skipped layer of
the exited tokens (ridge maps + W4A16 K/V projection + cache write). The
default workload is the GPT-2-small-shape prefill: 4096 tokens, d = 768,
12 layers, exit check at layer 4, fill of layers 5..12. Inputs are seeded
synthetic tensors; the ridge maps are fitted on the GPU (river_ridge_fit,
outside the timed region) from synthetic calibration states.

The timed region enqueues K steps back to back on one stream between two
events, after W warm-up steps. Each step uses the next of R rotating input
and output sets so that no set is still resident in the 256 MB MALL or the
L2 when it comes round again (inputs sit in HBM when the region starts).

Output: one JSON line with the metric, the roofline of the dominant kernel
(measured live with events on the launch stream) and the oracle's CPU time
on a bounded sample of the same workload.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import token_early_exit_amd as tee  # noqa: E402
from synth import get_config  # noqa: E402
from synth import generate as G  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 MFMA, TFLOP/s


def progress(msg):
    """One line on stderr per finished part (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=12, help="input/output sets cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle CPU time")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--projection-only", type=int, default=0,
                    help="only run this many projection-kernel launches (counter collection)")
    ap.add_argument("--decode-only", choices=["2", "3D"], default=None,
                    help="only time the decode step of one decode workload (2: Llama-3.2-1B, "
                         "3D: Llama-3-8B) and print its figures")
    ap.add_argument("--router-fit-only", action="store_true",
                    help="only time router calibration (both shapes) and print its figures")
    return ap.parse_args()


class Workload:
    """The GPT-2-shape prefill step, with R rotating sets of tensors."""

    def __init__(self, R, dev="cuda"):
        cfg = self.cfg = get_config(1)
        e = self.e = cfg.route_layers[0]
        self.layers = list(range(e + 1, cfg.L + 1))
        self.nl = len(self.layers)
        n, d = cfg.n_tokens, cfg.d
        # drawn on the CPU (the same tensors the parity tests check), then moved
        hs = G.hidden_states(cfg, n, [e - 1, e])
        self.h_prev0, self.h_cur0 = hs[e - 1].to(dev), hs[e].to(dev)
        self.wd, self.wu = (t.to(dev) for t in G.router_weights(cfg, e))
        w = G.kv_weights(cfg, self.layers)
        self.wk = tuple(t.to(dev) for t in w["wk"]) + (cfg.group,)
        self.wv = tuple(t.to(dev) for t in w["wv"]) + (cfg.group,)
        self.slot = G.slots(cfg, device=dev)
        self.gamma = G.final_norm_gamma(cfg).to(dev)
        # the skipped layers' own K/V path: input RMSNorm, K/V bias, RoPE
        self.lgamma = G.layer_norm_gammas(cfg, self.layers).to(dev)
        self.bk, self.bv = (t.to(dev) for t in G.kv_biases(cfg, self.layers))
        self.rcos, self.rsin = (t.to(dev) for t in G.rope_tables(cfg, n))
        self.pos = torch.arange(n, dtype=torch.int32, device=dev)
        # ridge maps fitted on the GPU from the calibration pass
        X, Y = (t.to(dev) for t in G.calibration(cfg, e))
        self.maps = torch.empty((self.nl, d, d), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(tee.river_workspace_size(tee.OP_RIDGE_FIT, X.shape[0], d, d, self.nl,
                                                  tee.RIVER_BF16), dtype=torch.uint8, device=dev)
        t0 = time.perf_counter()
        tee.river_ridge_fit(X, Y, cfg.ridge_lambda, self.maps, workspace=ws)
        self.ridge_ms = (time.perf_counter() - t0) * 1e3
        del X, Y, ws
        # R rotating sets: states (perturbed copies), outputs, caches
        self.sets = []
        for r in range(R):
            hp = self.h_prev0.clone()
            hc = self.h_cur0.clone()
            kc = torch.zeros((self.nl, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim),
                             dtype=torch.bfloat16, device=dev)
            self.sets.append({
                "hp": hp, "hc": hc, "kc": kc, "vc": torch.zeros_like(kc),
                "mask": torch.empty(n, dtype=torch.uint8, device=dev),
                "cont": torch.empty(n, dtype=torch.int32, device=dev),
                "ext": torch.empty(n, dtype=torch.int32, device=dev),
                "counts": torch.zeros(2, dtype=torch.int32, device=dev),
                "out": torch.empty((n, d), dtype=torch.bfloat16, device=dev),
            })
        self.cws = torch.empty(max(256, tee.river_workspace_size(tee.OP_COMPACT, n)),
                               dtype=torch.uint8, device=dev)
        self.kws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, n, d, 0, 0, self.nl),
                               dtype=torch.uint8, device=dev)
        self.lws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL_LAYER, n, d, 0, 0, self.nl),
                               dtype=torch.uint8, device=dev)

    # the three calls of one step
    def route(self, s):
        cfg = self.cfg
        tee.river_route(s["hp"], s["hc"], s["mask"], w_down=self.wd, w_up=self.wu,
                        tau=cfg.tau, theta=cfg.theta)

    def compact(self, s):
        tee.river_compact(s["mask"], s["hc"], s["cont"], s["ext"], s["counts"], out=s["out"],
                          workspace=self.cws)

    def fill(self, s):
        cfg = self.cfg
        tee.river_kv_fill(s["hc"], self.slot, self.wk, self.wv, cfg.n_kv_heads, cfg.head_dim,
                          s["kc"], s["vc"], m_max=cfg.n_tokens, m_dev=s["counts"][1:],
                          row_idx=s["ext"], maps=self.maps, workspace=self.kws)

    def fill_projection_only(self, s):
        """The K/V projection kernel alone (identity map, same rows, same
        output slots): one launch of the kernel that dominates the step."""
        cfg = self.cfg
        tee.river_kv_fill(s["hc"], self.slot, self.wk, self.wv, cfg.n_kv_heads, cfg.head_dim,
                          s["kc"], s["vc"], m_max=cfg.n_tokens, m_dev=s["counts"][1:],
                          row_idx=s["ext"], maps=None)

    def fill_layer(self, s):
        """The fill through the layers' full K/V path (input RMSNorm, K/V
        bias and RoPE on K), same rows, maps and slots as ``fill``."""
        cfg = self.cfg
        tee.river_kv_fill_layer(s["hc"], self.slot, self.wk, self.wv, cfg.n_kv_heads, cfg.head_dim,
                                s["kc"], s["vc"], m_max=cfg.n_tokens, m_dev=s["counts"][1:],
                                row_idx=s["ext"], maps=self.maps, norm_gamma=self.lgamma,
                                norm_eps=1e-5, k_bias=self.bk, v_bias=self.bv, pos=self.pos,
                                rope_cos=self.rcos, rope_sin=self.rsin, workspace=self.lws)

    def exit_projection(self, s):
        """Final RMSNorm of the exited rows into their positions of ``out``
        (timed on its own: it is not one of the step's three calls)."""
        cfg = self.cfg
        tee.river_exit_projection(s["hc"], s["out"], m_max=cfg.n_tokens, m_dev=s["counts"][1:],
                                  row_idx=s["ext"], gamma=self.gamma, eps=1e-5)

    def step(self, i):
        s = self.sets[i % len(self.sets)]
        self.route(s)
        self.compact(s)
        self.fill(s)

    # algorithmic work of one step
    def work(self, n_exit):
        cfg = self.cfg
        n, d, b, hd = cfg.n_tokens, cfg.d, cfg.b, cfg.hd
        route_bytes = 2 * n * d * 2 + b * d * 2 + b * 2 + n * 1
        compact_bytes = n * 1 + n * 4 + 2 * 4 + 2 * n_exit * d * 2   # mask, indices, counts, exit rows
        fill_flops = n_exit * self.nl * (2 * d * d + 2 * 2 * d * hd)
        fill_bytes = (self.nl * d * d * 2 + self.nl * 2 * hd * (d // 2 + 2 * 2 * d // cfg.group)
                      + n_exit * d * 2 + self.nl * n_exit * d * 2 * 2
                      + self.nl * n_exit * 2 * hd * 2)
        return route_bytes, compact_bytes, fill_flops, fill_bytes


def time_region(fn, steps):
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def per_call_times(wl, steps):
    """Average duration of each call, each bracketed by its own events on
    the launch stream."""
    names = ("route", "compact", "fill")
    ev = {k: [] for k in names}
    torch.cuda.synchronize()
    for i in range(steps):
        s = wl.sets[i % len(wl.sets)]
        for k in names:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            getattr(wl, k)(s)
            b.record()
            ev[k].append((a, b))
    torch.cuda.synchronize()
    return {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}


def kernel_times(wl, launches):
    """Average duration of one call of each kind (route, the projection
    kernel alone, the exit projection, the whole fill with and without the
    layers' K/V path). ``launches`` calls of one
    kind (rotating sets) are captured into a HIP graph, and one replay is
    bracketed by two events on the stream it runs on; the total divided by
    the number of launches is the kernel's own duration plus the short
    dispatch gap between graph nodes, the figure a kernel trace reports as
    the average duration. The graph keeps host-side launch cost (the Python
    binding takes several microseconds per call) out of the figure, which
    matters for kernels shorter than that."""
    out = {}
    for k, fn in (("route", wl.route), ("projection", wl.fill_projection_only),
                  ("exit_projection", wl.exit_projection), ("fill", wl.fill),
                  ("fill_layer", wl.fill_layer)):
        for i in range(len(wl.sets)):
            fn(wl.sets[i])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(launches):
                fn(wl.sets[i % len(wl.sets)])
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out[k] = a.elapsed_time(b) / launches
        del g
    return out


class DecodeWorkload:
    """One generation step of the token-level exit loop on a decode shape:
    Llama-3.2-1B (64 tokens, checks after blocks 8..15, router off, tau_l at
    the midpoint of the two middle cosines of the tokens still running,
    identity fill) or Llama-3-8B (256 tokens, a router at every fourth block,
    tau off, theta_11 between the 13th and 14th largest probabilities,
    theta_31 = -inf and +inf elsewhere, near-identity maps). The thresholds
    come from the library's own cosines and probabilities."""

    def __init__(self, key, dev="cuda"):
        cfg = self.cfg = get_config(key)
        n = cfg.n_tokens
        layers = list(cfg.route_layers)
        need = sorted({l - 1 for l in layers} | set(layers))
        self.hs = G.hidden_states(cfg, n, need, device=dev)
        self.slot = G.slots(cfg, device=dev)
        w = G.kv_weights(cfg, list(range(1, cfg.L + 1)), device=dev)
        self.wk = tuple(w["wk"]) + (cfg.group,)
        self.wv = tuple(w["wv"]) + (cfg.group,)
        self.kc = torch.zeros((cfg.L, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim),
                              dtype=torch.bfloat16, device=dev)
        self.vc = torch.zeros_like(self.kc)
        self.ex = torch.empty(n, dtype=torch.int32, device=dev)
        # with room for the fills' split reduction (n <= 64)
        wsn = tee.river_workspace_size(tee.OP_DECODE_STEP, n, cfg.d, cfg.n_kv_heads * cfg.head_dim,
                                       0, cfg.L)
        self.ws = torch.empty(wsn, dtype=torch.uint8, device=dev)
        cos = torch.empty(n, device=dev)
        prob = torch.empty(n, device=dev)
        mask = torch.empty(n, dtype=torch.uint8, device=dev)
        alive = np.ones(n, bool)
        self.cks = []
        for l in layers:
            c = {"layer": l, "h_prev": self.hs[l - 1], "h_cur": self.hs[l]}
            if cfg.b:
                wd, wu = (t.to(dev) for t in G.router_weights(cfg, l))
                c["w_down"], c["w_up"] = wd, wu
                tee.river_route(self.hs[l - 1], self.hs[l], mask, w_down=wd, w_up=wu,
                                prob_out=prob)
                c["tau"] = -math.inf
                if l == cfg.extra["exit_early"]:
                    p = np.sort(prob.cpu().numpy())[::-1]
                    k = int(round(cfg.extra["early_frac"] * n))
                    c["theta"] = 0.5 * (p[k - 1] + p[k])
                    c["maps"] = G.near_identity_maps(cfg, cfg.L - l, device=dev)
                elif l == cfg.extra["exit_late"]:
                    c["theta"] = -math.inf
                    c["maps"] = G.near_identity_maps(cfg, cfg.L - l, tag="maps31", device=dev)
                else:
                    c["theta"] = math.inf
            else:
                tee.river_route(self.hs[l - 1], self.hs[l], mask, cos_out=cos)
                cv = cos.cpu().numpy()
                a = np.sort(cv[alive])
                m = len(a)
                c["tau"] = 0.5 * (a[(m - 1) // 2] + a[m // 2]) if m > 1 else -math.inf
                c["theta"] = -math.inf
                alive &= ~(cv > np.float32(c["tau"]))
            self.cks.append(c)
        torch.cuda.synchronize()

    def step(self, i=0):
        cfg = self.cfg
        tee.river_decode_step(self.cks, self.wk, self.wv, cfg.n_kv_heads, cfg.head_dim, self.slot,
                              self.kc, self.vc, self.ex, workspace=self.ws)


def decode_times(key, steps):
    """µs per decode step: eager (each call enqueues the step's kernels from
    the host) and replayed from one captured graph."""
    dw = DecodeWorkload(key)
    for _ in range(3):
        dw.step()
    torch.cuda.synchronize()
    eager = time_region(dw.step, steps) / steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dw.step()
    g.replay()
    torch.cuda.synchronize()
    graph = time_region(lambda i: g.replay(), steps) / steps
    ex = dw.ex.cpu().numpy()
    cfg = dw.cfg
    n_ck = len(dw.cks)
    # the launch sequence the library takes for this workload
    if cfg.n_tokens <= 1024 and n_ck <= (16 if cfg.b else 32):
        scores = "one route launch for all checkpoints" if cfg.b else "cosines of all checkpoints"
        plain = sum(c.get("maps") is None for c in dw.cks)
        if plain == n_ck:
            path = (f"{scores}, one decision workgroup, gather of the exit states, one projection "
                    "over all filled blocks")
        elif plain >= 2:
            path = (f"{scores}, one decision workgroup, gather of the exit states and one projection "
                    "for the checkpoints without maps, a fill per checkpoint with maps")
        else:
            path = f"{scores}, one decision workgroup, a fill per checkpoint"
    else:
        path = "per checkpoint: route, compact, fill"
    del g
    return {"tokens": cfg.n_tokens, "d": cfg.d, "blocks": cfg.L, "checkpoints": n_ck,
            "exits_per_checkpoint": [int((ex == c["layer"]).sum()) for c in dw.cks],
            "filled_token_layers": int(sum(cfg.L - e for e in ex)),
            "path": path, "eager_us": eager * 1e3, "graph_us": graph * 1e3}


def router_fit_times(key, n, epochs=100, batch=256):
    """One checkpoint's router trained on n synthetic calibration tokens
    (labels from the library's cosine test at 0.98), timed whole between two
    events: the page's setting of 100 epochs, Adam lr 1e-3."""
    cfg = get_config(key)
    k = cfg.route_layers[0]
    hk, hf = (t.to("cuda") for t in G.router_calibration(cfg, k, n, device="cuda"))
    y = torch.empty(n, dtype=torch.uint8, device="cuda")
    tee.river_route(hf, hk, y, tau=0.98)
    wd, wu = G.router_weights(cfg, k)
    W0 = wd.float().cuda()
    w0 = wu.float().cuda()
    ws = torch.empty(tee.river_workspace_size(tee.OP_ROUTER_FIT, n, cfg.d, cfg.b, batch, epochs),
                     dtype=torch.uint8, device="cuda")
    loss = torch.empty(epochs, device="cuda")
    W, w = W0.clone(), w0.clone()
    tee.river_router_fit(hk, y, W, w, epochs=1, batch=batch, loss_out=loss, workspace=ws)  # warm-up
    W, w = W0.clone(), w0.clone()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    tee.river_router_fit(hk, y, W, w, epochs=epochs, batch=batch, loss_out=loss, workspace=ws)
    host_ms = (time.perf_counter() - t0) * 1e3
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    steps = epochs * ((n + batch - 1) // batch)
    lo = loss.cpu().numpy()
    return {"tokens": n, "d": cfg.d, "b": cfg.b, "epochs": epochs, "batch": batch,
            "adam_steps": steps, "ms": ms, "us_per_step": ms * 1e3 / steps,
            "host_enqueue_ms": host_ms, "token_epochs_per_s": n * epochs / (ms * 1e-3),
            "converged_fraction": float(y.float().mean().item()),
            "loss_first_last_epoch": [float(lo[0]), float(lo[-1])]}


def fill_8b_prefill(reps=3):
    """The fill at the Llama-3-8B prefill shape (8192 tokens, d = 4096,
    8 x 128 KV heads, int4 group 128, near-identity maps): the 5% of tokens
    that exit at block 11 (410 rows, blocks 12..32) and the rest at block 31
    (7782 rows, block 32). ms per call averaged over ``reps`` calls between
    two events, and TFLOP/s on the algorithmic flops (map GEMM and
    projection)."""
    cfg = get_config(3)
    n, d = cfg.n_tokens, cfg.d
    nh = cfg.n_kv_heads * cfg.head_dim
    hs = G.hidden_states(cfg, n, [11, 31], device="cuda")
    slot = G.slots(cfg, device="cuda")
    n_early = int(round(cfg.extra["early_frac"] * n))
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3))
    early = torch.sort(perm[:n_early]).values.to(torch.int32).to("cuda")
    late = torch.sort(perm[n_early:]).values.to(torch.int32).to("cuda")
    out = {}
    for name, e, rows in (("exit_at_11", 11, early), ("exit_at_31", 31, late)):
        layers = list(range(e + 1, cfg.L + 1))
        nl = len(layers)
        w = G.kv_weights(cfg, layers, device="cuda")
        wk = tuple(w["wk"]) + (cfg.group,)
        wv = tuple(w["wv"]) + (cfg.group,)
        maps = G.near_identity_maps(cfg, nl, tag=f"maps{e}", device="cuda")
        m = rows.numel()
        kc = torch.empty((nl, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16,
                         device="cuda")
        vc = torch.empty_like(kc)
        ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, m, d, nh, 0, nl), dtype=torch.uint8,
                         device="cuda")

        def fill(i):
            tee.river_kv_fill(hs[e], slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=m,
                              row_idx=rows, maps=maps, workspace=ws)
        fill(0)
        torch.cuda.synchronize()
        ms = time_region(fill, reps) / reps
        flops = 2.0 * m * nl * (d * d + d * 2 * nh)
        out[name] = {"rows": m, "layers": nl, "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
                     "frac_of_bf16_peak": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
        del w, wk, wv, maps, kc, vc, ws
        torch.cuda.empty_cache()
    return out


def route_compact_8b(reps=20):
    """route and compact at the Llama-3-8B prefill shape (8192 tokens,
    d = 4096, router b = 128 at checkpoint 11): µs per call (graph of
    back-to-back calls between two events) and HBM GB/s on the algorithmic
    bytes (route: both state rows of every token and W_down; compact: the
    mask, the index lists and the exited rows read and written)."""
    cfg = get_config(3)
    n, d, b = cfg.n_tokens, cfg.d, cfg.b
    e = 11
    hs = G.hidden_states(cfg, n, [e - 1, e], device="cuda")
    wd, wu = (t.to("cuda") for t in G.router_weights(cfg, e))
    mask = torch.empty(n, dtype=torch.uint8, device="cuda")
    prob = torch.empty(n, device="cuda")
    tee.river_route(hs[e - 1], hs[e], mask, w_down=wd, w_up=wu, prob_out=prob)
    p = np.sort(prob.cpu().numpy())[::-1]
    k = int(round(cfg.extra["early_frac"] * n))
    theta = float(0.5 * (p[k - 1] + p[k]))
    cont = torch.empty(n, dtype=torch.int32, device="cuda")
    ext = torch.empty(n, dtype=torch.int32, device="cuda")
    counts = torch.empty(2, dtype=torch.int32, device="cuda")
    out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    cws = torch.empty(max(256, tee.river_workspace_size(tee.OP_COMPACT, n)), dtype=torch.uint8,
                      device="cuda")
    route = lambda i: tee.river_route(hs[e - 1], hs[e], mask, w_down=wd, w_up=wu, tau=-math.inf,
                                      theta=theta)
    compact = lambda i: tee.river_compact(mask, hs[e], cont, ext, counts, out=out, workspace=cws)
    res = {}
    for name, fn in (("route", route), ("compact", compact)):
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        res[name] = time_region(lambda i: g.replay(), 1) / reps
        del g
    ne = int(counts[1].item())
    route_b = 2 * n * d * 2 + b * d * 2 + b * 2 + n
    compact_b = n + 4 * n + 8 + 2 * ne * d * 2
    return {"tokens": n, "d": d, "exited": ne,
            "route_us": res["route"] * 1e3, "route_gbs": route_b / (res["route"] * 1e-3) / 1e9,
            "route_frac_hbm": route_b / (res["route"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "compact_us": res["compact"] * 1e3,
            "compact_gbs": compact_b / (res["compact"] * 1e-3) / 1e9,
            "route_compact_frac_hbm": (route_b + compact_b) / ((res["route"] + res["compact"]) * 1e-3)
                                      / 1e9 / HBM_PEAK_GBS}


def fill_long_context(reps=3):
    """The fill at the long-context prefill shape (d = 5120, exit after block
    16 of 64, the 30,704 rows between the first 16 and the last 2048 of a
    32K-token prompt, 48 filled layers, near-identity maps, int4 group 128,
    8 x 128 KV heads): the shape where the GEMMs fill the GPU. Whole fill
    and projection alone, each averaged over ``reps`` calls between two
    events."""
    cfg = get_config(4)
    e = 16
    layers = list(range(e + 1, cfg.L + 1))
    nl = len(layers)
    n, d = cfg.n_tokens, cfg.d
    h = G.hidden_states(cfg, n, [e], device="cuda")[e]
    slot = G.slots(cfg, device="cuda")
    w = G.kv_weights(cfg, layers, device="cuda")
    wk = tuple(w["wk"]) + (cfg.group,)
    wv = tuple(w["wv"]) + (cfg.group,)
    maps = G.near_identity_maps(cfg, nl, device="cuda")
    rows = torch.arange(cfg.fill_lo, n - cfg.fill_tail, dtype=torch.int32, device="cuda")
    m = rows.numel()
    kc = torch.empty((nl, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16,
                     device="cuda")
    vc = torch.empty_like(kc)
    # with room for the projection on dequantised weights
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, m, d, cfg.n_kv_heads * cfg.head_dim, 0, nl),
                     dtype=torch.uint8, device="cuda")

    def fill(with_maps):
        tee.river_kv_fill(h, slot, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, vc, m_max=m,
                          row_idx=rows, maps=maps if with_maps else None, workspace=ws)

    out = {}
    for key, wm in (("fill_ms", True), ("projection_ms", False)):
        fill(wm)
        torch.cuda.synchronize()
        out[key] = time_region(lambda i: fill(wm), reps) / reps
    n_out = 2 * cfg.n_kv_heads * cfg.head_dim
    map_flops = 2.0 * m * d * d * nl
    proj_flops = 2.0 * m * d * n_out * nl
    map_ms = out["fill_ms"] - out["projection_ms"]
    del maps, ws, kc, vc
    torch.cuda.empty_cache()
    return {"rows": m, "d": d, "layers": nl, "n_out": n_out,
            "fill_ms": out["fill_ms"], "projection_ms": out["projection_ms"],
            "map_gemm_ms": map_ms,
            "map_gemm_tflops": map_flops / (map_ms * 1e-3) / 1e12,
            "map_gemm_frac_of_bf16_peak": map_flops / (map_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "projection_tflops": proj_flops / (out["projection_ms"] * 1e-3) / 1e12,
            "fill_tflops": (map_flops + proj_flops) / (out["fill_ms"] * 1e-3) / 1e12,
            "fill_frac_of_bf16_peak": (map_flops + proj_flops) / (out["fill_ms"] * 1e-3) / 1e12
                                      / MFMA_BF16_PEAK_TFLOPS,
            "exited_tokens_per_s": m / (out["fill_ms"] * 1e-3)}


def router_fit_all():
    return {
        "gpt2-small shape: checkpoint 4, 2048 calibration tokens": router_fit_times(1, 2048),
        "llama3-8b shape: checkpoint 3, 8192 calibration tokens": router_fit_times(3, 8192),
    }


def source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# the projection kernel's own code: the kernel and its launch (w4gemm.h), the
# dequantization and scheduling helpers (gemm.h) and the device helpers
# (common.h)
KERNEL_SOURCES = ["token_early_exit_amd/csrc/w4gemm.h", "token_early_exit_amd/csrc/gemm.h",
                  "token_early_exit_amd/csrc/common.h"]


def measured_traffic():
    """HBM bytes per launch of the projection kernel from the committed
    rocprofv3 counter summary, or None when the kernel sources changed since
    the counters were taken."""
    f = os.path.join(ROOT, "profiles", "kv_projection_gpt2_traffic.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash(KERNEL_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, target_s):
    """The oracle (float64 NumPy, as it stands) on whole steps of the same
    workload, repeated until about ``target_s`` seconds of CPU time."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    cfg = wl.cfg
    hp = wl.h_prev0.double().cpu().numpy()
    hc = wl.h_cur0.double().cpu().numpy()
    wd = wl.wd.double().cpu().numpy()
    wu = wl.wu.double().cpu().numpy()
    maps = wl.maps.float().cpu().numpy()
    wk = {"q": wl.wk[0].cpu().numpy(), "scale": wl.wk[1].double().cpu().numpy(),
          "zero": wl.wk[2].double().cpu().numpy(), "group": cfg.group}
    wv = {"q": wl.wv[0].cpu().numpy(), "scale": wl.wv[1].double().cpu().numpy(),
          "zero": wl.wv[2].double().cpu().numpy(), "group": cfg.group}
    slot = wl.slot.cpu().numpy()
    kc = np.zeros((wl.nl, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim))
    steps, exited = 0, 0
    t0 = time.perf_counter()
    while True:
        _, _, mask, _ = O.route(hp, hc, None, 1e-6, wd, wu, cfg.tau, cfg.theta)
        res = O.compact(mask, hc, None, np.zeros_like(hc))
        ex = res["exit_idx"]
        O.kv_fill(hc, ex, len(ex), slot, maps, wk, wv, cfg.n_kv_heads, cfg.head_dim, kc, kc)
        steps += 1
        exited += len(ex)
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    return {"value": exited / el, "unit": "exited tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{steps} whole steps of the same workload (route of {cfg.n_tokens} tokens, "
                      f"compact, kv_fill of {len(ex)} exited tokens x {wl.nl} layers) in {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only (no sharding across GPUs): --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    tee.load()
    torch.cuda.set_device(0)
    if args.copy_probe_mb:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE calibration
        n = args.copy_probe_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
        return
    if args.router_fit_only:
        print(json.dumps({"router_fit": router_fit_all()}))
        return
    if args.decode_only:
        key = 2 if args.decode_only == "2" else "3D"
        print(json.dumps({"decode_step": decode_times(key, 20)}))
        return
    wl = Workload(args.rotate)
    if args.projection_only:
        for i in range(len(wl.sets)):
            wl.step(i)            # the exit lists of every set
        torch.cuda.synchronize()
        for i in range(args.projection_only):
            wl.fill_projection_only(wl.sets[i % len(wl.sets)])
        torch.cuda.synchronize()
        print(json.dumps({"projection_launches": args.projection_only,
                          "exited": int(wl.sets[0]["counts"][1].item())}))
        return

    # warm-up, then the timed region
    for i in range(args.warmup):
        wl.step(i)
    ms_total = time_region(wl.step, args.steps)
    ms_step = ms_total / args.steps
    n_exit = int(wl.sets[0]["counts"][1].item())
    progress(f"{args.steps} timed steps: {ms_step * 1e3:.1f} us per step")
    calls = per_call_times(wl, max(20, args.steps // 4))
    kern = kernel_times(wl, max(50, args.steps))
    progress("per-call and per-kernel timing done")

    route_b, compact_b, fill_f, fill_b = wl.work(n_exit)
    value = n_exit / (ms_step * 1e-3)
    # dominant kernel: the W4A16 K/V projection GEMM with the cache write
    # (w4_gemm_kernel<128, cache>); algorithmic flops per launch =
    # exited rows x layers x 2 x d x (2 n_kv_heads head_dim)
    cfg = wl.cfg
    proj_flops = n_exit * wl.nl * 2 * cfg.d * 2 * cfg.hd
    ach = proj_flops / (kern["projection"] * 1e-3) / 1e12
    roof = {"kernel": "w4_gemm_kernel<128,cache> (kv_fill K/V projection)", "bound": "mfma",
            "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / MFMA_BF16_PEAK_TFLOPS, "traffic": measured_traffic(),
            "flops_per_launch": proj_flops, "avg_launch_us": kern["projection"] * 1e3}

    # exit projection: reads and writes each exited row once, plus its two
    # indices (exit_idx entry, and the identity row id)
    ep_bytes = n_exit * (2 * cfg.d * 2 + 4)
    ep_gbs = ep_bytes / (kern["exit_projection"] * 1e-3) / 1e9
    exit_proj = {"kernel": "exit_proj_kernel<bf16,2> (final RMSNorm + scatter)", "bound": "hbm",
                 "avg_launch_us": kern["exit_projection"] * 1e3, "bytes_per_launch": ep_bytes,
                 "achieved": ep_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": ep_gbs / HBM_PEAK_GBS}

    line = {
        "metric": "exited tokens/s (route+compact+kv_fill)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gpt2-small-shape prefill: 4096 tokens, d=768, L=12, exit check "
                               "at layer 4 (tau=0.9, theta=0.5, router b=128), fill of layers "
                               "5-12 through ridge maps and int4 (group 64) K/V, 12x64 KV heads",
                   "exited_per_step": n_exit, "rotating_sets": args.rotate},
        "breakdown_us": {k: v * 1e3 for k, v in calls.items()},
        "route_kernel_us": kern["route"] * 1e3,
        "fill_tflops": fill_f / (calls["fill"] * 1e-3) / 1e12,
        "route_gbs": route_b / (calls["route"] * 1e-3) / 1e9,
        "compact_gbs": compact_b / (calls["compact"] * 1e-3) / 1e9,
        "ridge_fit_ms_once": wl.ridge_ms,
        "exit_projection": exit_proj,
        "fill_layer": {"parts": "input RMSNorm + K/V bias + RoPE on K (head_dim 64), ridge maps",
                       "avg_call_us": kern["fill_layer"] * 1e3,
                       "plain_fill_avg_call_us": kern["fill"] * 1e3,
                       "overhead_us": (kern["fill_layer"] - kern["fill"]) * 1e3},
        "roofline": roof,
    }
    line["decode_step"] = {
        "llama3.2-1b decode: 64 tokens, d=2048, checks after blocks 8..15 (router off), identity fill":
            decode_times(2, 50),
        "llama3-8b decode: 256 tokens, d=4096, 8 router checkpoints, maps for the exits at 11 and 31":
            decode_times("3D", 20),
    }
    progress("decode steps done")
    line["router_fit"] = router_fit_all()
    progress("router calibration done")
    line["fill_long_context"] = fill_long_context()
    progress("long-context fill done")
    line["route_compact_8b_prefill"] = route_compact_8b()
    line["fill_8b_prefill"] = fill_8b_prefill()
    progress("8B route, compact and fill done")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        progress("cpu baseline done")
    print(json.dumps(line))


if __name__ == "__main__":
    main()
