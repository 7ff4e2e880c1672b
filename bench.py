"""Benchmark of the per-token exit-and-KV-fill step on one MI355X.

A step is one pass of the hot path over one batch: the exit decision
(river_route, or a positional rule), the split of the batch
(river_compact), and the K/V fill of every skipped layer of the exited
tokens (river_kv_fill: ridge maps, W4A16 K/V projection, cache write).

Headline workload: RidgeFill's long-context prefill, the largest workload
that fits one GPU: d = 5120, 64 blocks, split after block 16, 65,536 tokens
(``--tokens 32768`` for the shorter run). The tokens between the first 16
and the last 2048 exit at the split (a positional rule: a mask compacted
into the list of rows to fill) and fill blocks 17..64 through 48 ridge maps
of 5120 x 5120, fitted on the GPU by river_ridge_fit from 16,384 synthetic
calibration tokens (timed on its own, outside the step). Every input is
seeded synthetic data resident in HBM when the timed region starts; at this
size nothing of one step (2.5 GB of maps, 0.65 GB of states, 13 GB of cache
writes) is still in the 256 MB MALL when the next one starts.

The timed region enqueues K steps back to back on one stream between two
HIP events, after W warm-up steps. The other workloads (the Llama-3-8B
prefill step over all its checkpoints, the GPT-2-shape step, the decode
steps, router calibration, the route and compaction with cold inputs) are
reported as extra keys of the same JSON line.

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
INF = math.inf


def progress(msg):
    """One line on stderr per finished part (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--tokens", type=int, default=65536, choices=[32768, 65536],
                    help="context length of the long-context prefill (the headline workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    choices=["long", "8b", "8b-folded", "gpt2", "route-compact", "decode2", "decode3D",
                             "decode3D-folded", "router-fit", "copy"],
                    help="run one workload only and print its figures (profiling runs)")
    ap.add_argument("--copy-probe-mb", type=int, default=256,
                    help="with --only copy: a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--rotate", type=int, default=12, help="GPT-2-shape input/output sets cycled through")
    return ap.parse_args()


def time_region(fn, steps):
    """ms for ``steps`` calls of fn(i), between two events on the current stream."""
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def graph_time(fn, launches, sets=1):
    """ms per call of fn(i): ``launches`` calls captured into one HIP graph and
    one replay bracketed by two events on the stream it runs on (the host's
    per-call cost stays out of the figure)."""
    for i in range(sets):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / launches


def kv_tuple(w, key, group):
    return tuple(w[key]) + (group,)


# ----------------------------------------------------------- workloads

class LongContextWorkload:
    """RidgeFill's long-context prefill: d = 5120, 64 blocks, 8 x 128 K/V
    heads (int4, group 128), heavy-tailed states; the rows between the first
    16 and the last 2048 tokens exit after block 16 and fill blocks 17..64.

    One step: river_compact of the positional mask (the list of rows to fill
    and the counts), then river_kv_fill of those rows with the 48 ridge maps
    and the workspace river_workspace_size gives for every layer and the
    projection (x_hat of all 48 layers, the dequantised K/V weights).

    maps: None fits the 48 maps on the GPU with river_ridge_fit from the
    16,384 calibration tokens (timed as ``ridge_ms``); otherwise the given
    [48][5120][5120] bf16 maps (or any object whose [l] is a map, turned into
    one tensor here)."""

    def __init__(self, N=65536, maps=None, dev="cuda"):
        cfg = self.cfg = get_config(4, n_tokens=N, n_slots=N)
        e = self.e = cfg.route_layers[0]
        self.layers = list(range(e + 1, cfg.L + 1))
        self.nl = nl = len(self.layers)
        d = cfg.d
        self.n_out = cfg.n_kv_heads * cfg.head_dim
        self.h = G.hidden_states(cfg, N, [e], device=dev)[e]
        self.slot = G.slots(cfg, device=dev)
        w = G.kv_weights(cfg, self.layers, device=dev)
        self.wk, self.wv = kv_tuple(w, "wk", cfg.group), kv_tuple(w, "wv", cfg.group)
        pos = torch.arange(N)
        self.mask = ((pos >= cfg.fill_lo) & (pos < N - cfg.fill_tail)).to(torch.uint8).to(dev)
        self.m = int(self.mask.sum())
        self.ridge_ms = None
        self.n_calib = cfg.n_calib
        if maps is None:
            X, Y = G.calibration(cfg, e, device=dev)
            self.maps = torch.empty((nl, d, d), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(tee.river_workspace_size(tee.OP_RIDGE_FIT, X.shape[0], d, d, nl,
                                                      tee.RIVER_BF16), dtype=torch.uint8, device=dev)
            tee.river_ridge_fit(X, Y, cfg.ridge_lambda, self.maps, workspace=ws)   # warm-up
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            tee.river_ridge_fit(X, Y, cfg.ridge_lambda, self.maps, workspace=ws)   # synchronous
            self.ridge_ms = (time.perf_counter() - t0) * 1e3
            del X, Y, ws
        else:
            self.maps = maps if isinstance(maps, torch.Tensor) else torch.stack(
                [maps[l].to(dev) for l in range(nl)]).contiguous()
        self.kc = torch.zeros((nl, N, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device=dev)
        self.vc = torch.zeros_like(self.kc)
        self.cont = torch.empty(N, dtype=torch.int32, device=dev)
        self.ext = torch.empty(N, dtype=torch.int32, device=dev)
        self.counts = torch.zeros(2, dtype=torch.int32, device=dev)
        self.cws = torch.empty(max(256, tee.river_workspace_size(tee.OP_COMPACT, N)), dtype=torch.uint8,
                               device=dev)
        self.ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, self.m, d, self.n_out, 0, nl),
                              dtype=torch.uint8, device=dev)
        torch.cuda.empty_cache()

    def compact(self, i=0):
        tee.river_compact(self.mask, None, self.cont, self.ext, self.counts, workspace=self.cws)

    def fill(self, i=0, maps=True):
        cfg = self.cfg
        tee.river_kv_fill(self.h, self.slot, self.wk, self.wv, cfg.n_kv_heads, cfg.head_dim, self.kc,
                          self.vc, m_max=self.m, row_idx=self.ext, maps=self.maps if maps else None,
                          workspace=self.ws)

    def step(self, i=0):
        self.compact()
        self.fill()

    def fold(self):
        """F = deq([Wk; Wv]) M of the 48 maps, formed once (river_kv_fold)."""
        self.F, self.fold_ms = fold_maps(self.cfg, self.maps, self.wk, self.wv)

    def fill_folded(self, i=0):
        cfg = self.cfg
        tee.river_kv_fill_folded(self.h, self.slot, self.F, cfg.n_kv_heads, cfg.head_dim, self.kc, self.vc,
                                 m_max=self.m, row_idx=self.ext)

    def step_folded(self, i=0):
        self.compact()
        self.fill_folded()

    def flops(self):
        """(the maps over every row, the projection of every row, the
        product of the weights and the maps): the fill runs the last two
        (through F = deq([Wk; Wv]) . M per layer); the two-phase form would
        run the first two."""
        d = self.cfg.d
        map_f = 2.0 * self.m * d * d * self.nl
        proj_f = 2.0 * self.m * d * 2 * self.n_out * self.nl
        prod_f = 2.0 * 2 * self.n_out * d * d * self.nl
        return map_f, proj_f, prod_f


class Prefill8BWorkload:
    """The Llama-3-8B prefill step: 8192 tokens, d = 4096, 32 blocks, a
    router (b = 128) at every fourth block {3, 7, ..., 31}, 8 x 128 K/V
    heads (int4, group 128). The cosine test is off; theta at block 11 puts
    about 5% of the tokens out, theta at block 31 is -inf (every token still
    running exits) and +inf elsewhere.

    One step, checkpoint by checkpoint: river_route over the tokens still
    running, river_compact (index lists, counts, the gather of the continuing
    rows with their token ids, and the exit scatter of the exited rows to
    their token positions), and river_kv_fill of the exited rows at blocks
    11 (blocks 12..32 through 21 ridge maps) and 31 (block 32, one map),
    with the row count read on the device. The states of the checkpoints
    after 11 are those of the continuing tokens, in their compacted order, as
    the backbone would produce them (gathered once here).

    theta11: None takes the midpoint between the library's own 410th and
    411th largest probabilities; tests pass the oracle's. maps11, maps31:
    None fits them on the GPU from the 8192 calibration tokens."""

    CKS = tuple(range(3, 32, 4))

    def __init__(self, theta11=None, maps11=None, maps31=None, dev="cuda"):
        cfg = self.cfg = get_config(3)
        n, d = cfg.n_tokens, cfg.d
        self.n, self.d = n, d
        self.e1, self.e2 = cfg.extra["exit_early"], cfg.extra["exit_late"]
        need = sorted({c - 1 for c in self.CKS} | set(self.CKS))
        hs = G.hidden_states(cfg, n, need, device=dev)
        self.routers = {c: G.router_weights(cfg, c, device=dev) for c in self.CKS}
        self.n_out = cfg.n_kv_heads * cfg.head_dim
        layers = list(range(self.e1 + 1, cfg.L + 1))             # blocks 12..32
        w = G.kv_weights(cfg, layers, device=dev)
        self.wk1, self.wv1 = kv_tuple(w, "wk", cfg.group), kv_tuple(w, "wv", cfg.group)
        late = cfg.L - self.e2                                    # block 32 only
        self.wk2 = tuple(t[-late:].contiguous() for t in w["wk"]) + (cfg.group,)
        self.wv2 = tuple(t[-late:].contiguous() for t in w["wv"]) + (cfg.group,)
        self.ridge_ms = None
        if maps11 is None or maps31 is None:
            t_ms = 0.0
            fitted = []
            for e in (self.e1, self.e2):
                X, Y = G.calibration(cfg, e, device=dev)
                M = torch.empty((Y.shape[0], d, d), dtype=torch.bfloat16, device=dev)
                ws = torch.empty(tee.river_workspace_size(tee.OP_RIDGE_FIT, X.shape[0], d, d, Y.shape[0],
                                                          tee.RIVER_BF16), dtype=torch.uint8, device=dev)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                tee.river_ridge_fit(X, Y, cfg.ridge_lambda, M, workspace=ws)
                t_ms += (time.perf_counter() - t0) * 1e3
                fitted.append(M)
                del X, Y, ws
            maps11, maps31 = fitted
            self.ridge_ms = t_ms
        self.maps = {self.e1: maps11.to(dev).contiguous(), self.e2: maps31.to(dev).contiguous()}
        self.slot = G.slots(cfg, device=dev)                     # positions
        self.kc = torch.zeros((cfg.L, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16,
                              device=dev)
        self.vc = torch.zeros_like(self.kc)
        self.out = torch.zeros((n, d), dtype=torch.bfloat16, device=dev)
        # thresholds
        self.theta = {c: INF for c in self.CKS}
        self.theta[self.e2] = -INF
        if theta11 is None:
            prob = torch.empty(n, device=dev)
            mask = torch.empty(n, dtype=torch.uint8, device=dev)
            wd, wu = self.routers[self.e1]
            tee.river_route(hs[self.e1 - 1], hs[self.e1], mask, w_down=wd, w_up=wu, prob_out=prob)
            p = np.sort(prob.cpu().numpy())[::-1]
            k = int(round(cfg.extra["early_frac"] * n))
            theta11 = float(0.5 * (p[k - 1] + p[k]))
        self.theta[self.e1] = theta11
        # per checkpoint: states of the running tokens, their token ids, and
        # the step's outputs
        self.ck = {}
        ids = torch.arange(n, dtype=torch.int32, device=dev)
        running = None                                 # None: every token, identity order
        for c in self.CKS:
            if running is None:
                hp, hc, rid = hs[c - 1], hs[c], None
            else:
                li = running.long()
                hp, hc, rid = hs[c - 1][li].contiguous(), hs[c][li].contiguous(), running
            nc = hc.shape[0]
            s = {"hp": hp, "hc": hc, "ids": rid, "n": nc,
                 "mask": torch.empty(nc, dtype=torch.uint8, device=dev),
                 "cont": torch.empty(nc, dtype=torch.int32, device=dev),
                 "ext": torch.empty(nc, dtype=torch.int32, device=dev),
                 "counts": torch.zeros(2, dtype=torch.int32, device=dev),
                 "h_cont": torch.empty((nc, d), dtype=torch.bfloat16, device=dev),
                 "ids_cont": torch.empty(nc, dtype=torch.int32, device=dev),
                 "cws": torch.empty(max(256, tee.river_workspace_size(tee.OP_COMPACT, nc)),
                                    dtype=torch.uint8, device=dev)}
            if c in self.maps:
                nl = self.maps[c].shape[0]
                s["fws"] = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, nc, d, self.n_out, 0, nl),
                                       dtype=torch.uint8, device=dev)
                s["slot"] = self.slot if rid is None else rid   # slot of each row = its token position
            self.ck[c] = s
            # the decision at this checkpoint sets who runs on
            self.route(c)
            self.compact(c)
            nc_cont = int(s["counts"][0].item())
            if nc_cont < nc:
                running = s["ids_cont"][:nc_cont].clone() if rid is not None else s["cont"][:nc_cont].clone()
        self.exits = {c: int(self.ck[c]["counts"][1].item()) for c in self.CKS}
        del hs
        torch.cuda.empty_cache()

    def route(self, c):
        s = self.ck[c]
        wd, wu = self.routers[c]
        tee.river_route(s["hp"], s["hc"], s["mask"], w_down=wd, w_up=wu, tau=-INF, theta=self.theta[c])

    def compact(self, c):
        s = self.ck[c]
        tee.river_compact(s["mask"], s["hc"], s["cont"], s["ext"], s["counts"], row_ids=s["ids"],
                          h_cont=s["h_cont"], row_ids_cont=s["ids_cont"], out=self.out,
                          workspace=s["cws"])

    def fold(self):
        """From now on the fills run through the folded products F =
        deq([Wk; Wv]) M of each exit block's maps (formed here, once)."""
        self.F, self.fold_ms = {}, 0.0
        for c in self.maps:
            wk, wv = (self.wk1, self.wv1) if c == self.e1 else (self.wk2, self.wv2)
            self.F[c], ms = fold_maps(self.cfg, self.maps[c], wk, wv)
            self.fold_ms += ms

    def fill(self, c):
        s = self.ck[c]
        cfg = self.cfg
        wk, wv = (self.wk1, self.wv1) if c == self.e1 else (self.wk2, self.wv2)
        nl = self.maps[c].shape[0]
        if getattr(self, "F", None) is not None:
            tee.river_kv_fill_folded(s["hc"], s["slot"], self.F[c], cfg.n_kv_heads, cfg.head_dim,
                                     self.kc[cfg.L - nl:], self.vc[cfg.L - nl:], m_max=s["n"],
                                     m_dev=s["counts"][1:], row_idx=s["ext"])
            return
        tee.river_kv_fill(s["hc"], s["slot"], wk, wv, cfg.n_kv_heads, cfg.head_dim, self.kc[cfg.L - nl:],
                          self.vc[cfg.L - nl:], m_max=s["n"], m_dev=s["counts"][1:], row_idx=s["ext"],
                          maps=self.maps[c], workspace=s["fws"])

    def step(self, i=0):
        for c in self.CKS:
            self.route(c)
            self.compact(c)
            if c in self.maps:
                self.fill(c)

    def work(self):
        """Algorithmic bytes of route and compaction, fill flops, per step."""
        d, b = self.d, self.cfg.b
        rb = cb = 0
        ff = 0.0
        for c in self.CKS:
            s = self.ck[c]
            nc, ne = s["n"], self.exits[c]
            rb += 2 * nc * d * 2 + b * d * 2 + b * 2 + nc
            cb += nc + 4 * nc + 8 + (4 * nc if s["ids"] is not None else 0)
            cb += 2 * (nc - ne) * d * 2 + 4 * (nc - ne)          # continuing rows gathered, their ids
            cb += 2 * ne * d * 2                                  # exited rows scattered
            if c in self.maps:
                ff += self.fill_flops(c)
        return rb, cb, ff

    def fill_flops(self, c):
        """Flops of the fill at c as it runs: the map and the projection, or
        the projection through F once folded."""
        ne, nl, d = self.exits[c], self.maps[c].shape[0], self.d
        if getattr(self, "F", None) is not None:
            return 2.0 * ne * nl * d * 2 * self.n_out
        return 2.0 * ne * nl * (d * d + d * 2 * self.n_out)


class Gpt2Workload:
    """The GPT-2-small-shape prefill step, with R rotating sets of tensors:
    4096 tokens, d = 768, 12 layers, exit check at layer 4 (tau = 0.9,
    theta = 0.5, router b = 128), fill of layers 5..12 through ridge maps
    and int4 (group 64) K/V, 12 x 64 heads, the exit count on the device."""

    def __init__(self, R, maps=None, dev="cuda"):
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
        self.lgamma = G.layer_norm_gammas(cfg, self.layers).to(dev)
        self.bk, self.bv = (t.to(dev) for t in G.kv_biases(cfg, self.layers))
        self.rcos, self.rsin = (t.to(dev) for t in G.rope_tables(cfg, n))
        self.pos = torch.arange(n, dtype=torch.int32, device=dev)
        self.ridge_ms = None
        if maps is None:
            X, Y = (t.to(dev) for t in G.calibration(cfg, e))
            self.maps = torch.empty((self.nl, d, d), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(tee.river_workspace_size(tee.OP_RIDGE_FIT, X.shape[0], d, d, self.nl,
                                                      tee.RIVER_BF16), dtype=torch.uint8, device=dev)
            t0 = time.perf_counter()
            tee.river_ridge_fit(X, Y, cfg.ridge_lambda, self.maps, workspace=ws)
            self.ridge_ms = (time.perf_counter() - t0) * 1e3
            del X, Y, ws
        else:
            self.maps = maps.to(dev).contiguous()
        self.sets = []
        for r in range(R):
            kc = torch.zeros((self.nl, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim),
                             dtype=torch.bfloat16, device=dev)
            self.sets.append({
                "hp": self.h_prev0.clone(), "hc": self.h_cur0.clone(), "kc": kc, "vc": torch.zeros_like(kc),
                "mask": torch.empty(n, dtype=torch.uint8, device=dev),
                "cont": torch.empty(n, dtype=torch.int32, device=dev),
                "ext": torch.empty(n, dtype=torch.int32, device=dev),
                "counts": torch.zeros(2, dtype=torch.int32, device=dev),
                "out": torch.empty((n, d), dtype=torch.bfloat16, device=dev),
                "h_cont": torch.empty((n, d), dtype=torch.bfloat16, device=dev),
            })
        self.cws = torch.empty(max(256, tee.river_workspace_size(tee.OP_COMPACT, n)),
                               dtype=torch.uint8, device=dev)
        self.kws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL, n, d, 0, 0, self.nl),
                               dtype=torch.uint8, device=dev)
        self.lws = torch.empty(tee.river_workspace_size(tee.OP_KV_FILL_LAYER, n, d, 0, 0, self.nl),
                               dtype=torch.uint8, device=dev)

    def route(self, s):
        cfg = self.cfg
        tee.river_route(s["hp"], s["hc"], s["mask"], w_down=self.wd, w_up=self.wu,
                        tau=cfg.tau, theta=cfg.theta)

    def compact(self, s):
        """Index lists, counts, the gather of the continuing rows and the exit
        scatter of the exited rows."""
        tee.river_compact(s["mask"], s["hc"], s["cont"], s["ext"], s["counts"], h_cont=s["h_cont"],
                          out=s["out"], workspace=self.cws)

    def fill(self, s):
        cfg = self.cfg
        tee.river_kv_fill(s["hc"], self.slot, self.wk, self.wv, cfg.n_kv_heads, cfg.head_dim,
                          s["kc"], s["vc"], m_max=cfg.n_tokens, m_dev=s["counts"][1:],
                          row_idx=s["ext"], maps=self.maps, workspace=self.kws)

    def fill_projection_only(self, s):
        cfg = self.cfg
        tee.river_kv_fill(s["hc"], self.slot, self.wk, self.wv, cfg.n_kv_heads, cfg.head_dim,
                          s["kc"], s["vc"], m_max=cfg.n_tokens, m_dev=s["counts"][1:],
                          row_idx=s["ext"], maps=None)

    def fill_layer(self, s):
        cfg = self.cfg
        tee.river_kv_fill_layer(s["hc"], self.slot, self.wk, self.wv, cfg.n_kv_heads, cfg.head_dim,
                                s["kc"], s["vc"], m_max=cfg.n_tokens, m_dev=s["counts"][1:],
                                row_idx=s["ext"], maps=self.maps, norm_gamma=self.lgamma,
                                norm_eps=1e-5, k_bias=self.bk, v_bias=self.bv, pos=self.pos,
                                rope_cos=self.rcos, rope_sin=self.rsin, workspace=self.lws)

    def exit_projection(self, s):
        cfg = self.cfg
        tee.river_exit_projection(s["hc"], s["out"], m_max=cfg.n_tokens, m_dev=s["counts"][1:],
                                  row_idx=s["ext"], gamma=self.gamma, eps=1e-5)

    def step(self, i):
        s = self.sets[i % len(self.sets)]
        self.route(s)
        self.compact(s)
        self.fill(s)

    def fold(self):
        """F = deq([Wk; Wv]) M of the 8 maps, formed once (river_kv_fold)."""
        self.F, self.fold_ms = fold_maps(self.cfg, self.maps, self.wk, self.wv)

    def fill_folded(self, s):
        cfg = self.cfg
        tee.river_kv_fill_folded(s["hc"], self.slot, self.F, cfg.n_kv_heads, cfg.head_dim, s["kc"], s["vc"],
                                 m_max=cfg.n_tokens, m_dev=s["counts"][1:], row_idx=s["ext"])

    def step_folded(self, i):
        s = self.sets[i % len(self.sets)]
        self.route(s)
        self.compact(s)
        self.fill_folded(s)

    def work(self, n_exit):
        cfg = self.cfg
        n, d, b, hd = cfg.n_tokens, cfg.d, cfg.b, cfg.hd
        route_bytes = 2 * n * d * 2 + b * d * 2 + b * 2 + n
        # mask, index lists, counts, continuing rows gathered, exited rows scattered
        compact_bytes = n + 4 * n + 8 + 2 * (n - n_exit) * d * 2 + 2 * n_exit * d * 2
        fill_flops = n_exit * self.nl * (2 * d * d + 2 * 2 * d * hd)
        return route_bytes, compact_bytes, fill_flops


def fold_maps(cfg, maps, wk, wv, dev="cuda"):
    """F = deq([Wk; Wv]) . M for each layer of maps (river_kv_fold), and the
    milliseconds it took (once per fitted map, off the step)."""
    nl, d = maps.shape[0], maps.shape[1]
    n_out = cfg.n_kv_heads * cfg.head_dim
    F = torch.empty((nl, 2 * n_out, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(tee.river_workspace_size(tee.OP_KV_FOLD, 0, d, n_out, 0, nl), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tee.river_kv_fold(wk, wv, cfg.n_kv_heads, cfg.head_dim, F, maps=maps, workspace=ws)
    torch.cuda.synchronize()
    return F, (time.perf_counter() - t0) * 1e3


def fold_checkpoints(cfg, cks, wk, wv, dev="cuda"):
    """Folded products for every decode checkpoint with maps (blocks e+1..L
    of the weights), set as the checkpoint's "folded"; total milliseconds."""
    t = 0.0
    for c in cks:
        if c.get("maps") is None:
            continue
        e = c["layer"]
        sub = lambda w: tuple(x[e:] for x in w[:3]) + (w[3],)
        c["folded"], ms = fold_maps(cfg, c["maps"], sub(wk), sub(wv), dev)
        t += ms
    return t


class DecodeWorkload:
    """One generation step of the token-level exit loop on a decode shape:
    Llama-3.2-1B (64 tokens, checks after blocks 8..15, router off, tau_l at
    the midpoint of the two middle cosines of the tokens still running,
    identity fill) or Llama-3-8B (256 tokens, a router at every fourth block,
    tau off, theta_11 between the 13th and 14th largest probabilities,
    theta_31 = -inf and +inf elsewhere, near-identity maps). The thresholds
    come from the library's own cosines and probabilities."""

    def __init__(self, key, folded=False, dev="cuda"):
        cfg = self.cfg = get_config(key)
        n = cfg.n_tokens
        layers = list(cfg.route_layers)
        self.fold_ms = None
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
        if folded:
            self.fold_ms = fold_checkpoints(cfg, self.cks, self.wk, self.wv, dev)
        torch.cuda.synchronize()

    def step(self, i=0):
        cfg = self.cfg
        tee.river_decode_step(self.cks, self.wk, self.wv, cfg.n_kv_heads, cfg.head_dim, self.slot,
                              self.kc, self.vc, self.ex, workspace=self.ws)


# ------------------------------------------------------------ measurements

def decode_times(key, steps, folded=False):
    """µs per decode step: eager (each call enqueues the step's kernels from
    the host) and replayed from one captured graph. folded: the checkpoints
    with maps fill through river_kv_fold's products, formed beforehand."""
    dw = DecodeWorkload(key, folded=folded)
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
    if cfg.n_tokens <= 1024 and n_ck <= (16 if cfg.b else 32):
        if cfg.b:
            scores = ("the routes of all checkpoints in two halves of d per token group, their sum"
                      if cfg.d % 512 == 0 else "one route launch for all checkpoints")
        else:
            scores = "cosines of all checkpoints"
        plain = sum(c.get("maps") is None for c in dw.cks)
        # the fills: one for the checkpoints without maps when there are two
        # or more of them, one per other checkpoint; from two on the first
        # of the others runs on a second stream
        fills = (1 if plain >= 2 else plain) + (n_ck - plain)
        two = " (the first of them on a second stream)" if fills >= 2 else ""
        if plain == n_ck:
            path = (f"{scores}, one decision workgroup, gather of the exit states, one projection "
                    "over all filled blocks")
        elif plain >= 2:
            path = (f"{scores}, one decision workgroup, gather of the exit states and one projection "
                    f"for the checkpoints without maps, a fill per checkpoint with maps{two}")
        else:
            path = f"{scores}, one decision workgroup, a fill per checkpoint{two}"
        if folded:
            path += "; the fills with maps through the folded products deq([Wk; Wv]) M"
    else:
        path = "per checkpoint: route, compact, fill"
    del g
    extra = {"fold_ms_once": dw.fold_ms} if folded else {}
    return {"tokens": cfg.n_tokens, "d": cfg.d, "blocks": cfg.L, "checkpoints": n_ck,
            "exits_per_checkpoint": [int((ex == c["layer"]).sum()) for c in dw.cks],
            "filled_token_layers": int(sum(cfg.L - e for e in ex)),
            "path": path, "eager_us": eager * 1e3, "graph_us": graph * 1e3, **extra}


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


def router_fit_all():
    return {
        "gpt2-small shape: checkpoint 4, 2048 calibration tokens": router_fit_times(1, 2048),
        "llama3-8b shape: checkpoint 3, 8192 calibration tokens": router_fit_times(3, 8192),
    }


def route_compact_8b_cold(reps=24, sets=6):
    """route and compact at one Llama-3-8B prefill checkpoint (8192 tokens,
    d = 4096, router b = 128, block 11, about 5% exit), with cold inputs:
    ``sets`` copies of the two state tensors (134 MB per set, 805 MB for
    six) are cycled, so a call's states are not in the 256 MB MALL. µs per
    call (a graph of back-to-back calls between two events) and HBM GB/s on
    the algorithmic bytes: route reads both state rows of every token, the
    router and writes the mask; compact reads the mask, writes the index
    lists and counts, gathers the continuing rows and scatters the exited
    ones (each row read and written once)."""
    cfg = get_config(3)
    n, d, b = cfg.n_tokens, cfg.d, cfg.b
    e = cfg.extra["exit_early"]
    hs = G.hidden_states(cfg, n, [e - 1, e], device="cuda")
    wd, wu = G.router_weights(cfg, e, device="cuda")
    mask = torch.empty(n, dtype=torch.uint8, device="cuda")
    prob = torch.empty(n, device="cuda")
    tee.river_route(hs[e - 1], hs[e], mask, w_down=wd, w_up=wu, prob_out=prob)
    p = np.sort(prob.cpu().numpy())[::-1]
    k = int(round(cfg.extra["early_frac"] * n))
    theta = float(0.5 * (p[k - 1] + p[k]))
    S = [(hs[e - 1].clone(), hs[e].clone()) for _ in range(sets)]
    del hs
    masks = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(sets)]
    cont = torch.empty(n, dtype=torch.int32, device="cuda")
    ext = torch.empty(n, dtype=torch.int32, device="cuda")
    counts = torch.empty(2, dtype=torch.int32, device="cuda")
    h_cont = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    cws = torch.empty(max(256, tee.river_workspace_size(tee.OP_COMPACT, n)), dtype=torch.uint8,
                      device="cuda")

    def route(i):
        hp, hc = S[i % sets]
        tee.river_route(hp, hc, masks[i % sets], w_down=wd, w_up=wu, tau=-INF, theta=theta)

    def compact(i):
        tee.river_compact(masks[i % sets], S[i % sets][1], cont, ext, counts, h_cont=h_cont, out=out,
                          workspace=cws)
    res = {}
    for name, fn in (("route", route), ("compact", compact)):
        res[name] = graph_time(fn, reps, sets)
    ne = int(counts[1].item())
    route_b = 2 * n * d * 2 + b * d * 2 + b * 2 + n
    compact_b = n + 4 * n + 8 + 2 * (n - ne) * d * 2 + 2 * ne * d * 2
    rt, ct = res["route"] * 1e-3, res["compact"] * 1e-3
    return {"tokens": n, "d": d, "exited": ne, "input_sets": sets,
            "route_us": rt * 1e6, "route_bytes": route_b, "route_gbs": route_b / rt / 1e9,
            "route_frac_hbm": route_b / rt / 1e9 / HBM_PEAK_GBS,
            "compact_us": ct * 1e6, "compact_bytes": compact_b, "compact_gbs": compact_b / ct / 1e9,
            "compact_frac_hbm": compact_b / ct / 1e9 / HBM_PEAK_GBS,
            "route_compact_frac_hbm": (route_b + compact_b) / (rt + ct) / 1e9 / HBM_PEAK_GBS}


def source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# the projection GEMM's own code: the 4-wave 256 x 256 kernel and its launch
# (gemm_quad.h), the 8-wave kernel it shares helpers with (gemm_big.h), the
# scheduling helpers and argument block (gemm.h), the device helpers
# (common.h)
GEMM_SOURCES = ["token_early_exit_amd/csrc/gemm_quad.h", "token_early_exit_amd/csrc/gemm_big.h",
                    "token_early_exit_amd/csrc/gemm.h", "token_early_exit_amd/csrc/common.h"]


def measured_traffic(name, sources):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter
    summary, or None when the kernel's sources changed since the counters
    were taken."""
    f = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash(sources):
        return None
    return t.get("hbm_bytes_per_launch")


# ------------------------------------------------------------ CPU baseline

def host_info():
    try:
        model = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")][0]
    except Exception:
        model = "unknown"
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('architecture')})"
                         for p in threadpool_info() if p.get("user_api") == "blas")
    except Exception:
        pass
    return model, blas


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def _w4np(w):
    q, s, z, group = w
    return {"q": q.cpu().numpy(), "scale": s.double().cpu().numpy(), "zero": z.double().cpu().numpy(),
            "group": group}


def _host_maps(maps):
    """The maps as float32 host arrays, layer by layer (copied before the
    oracle's clock starts; float32 holds the bf16 values exactly)."""
    return [maps[l].float().cpu().numpy() for l in range(maps.shape[0])]


def cpu_baseline_long(wl, rows=4096):
    """The oracle (float64 NumPy) on a fixed subset of the long-context
    workload: the positional compaction of all tokens, then the fill of the
    first ``rows`` of the rows to fill through all 48 layers. The time per
    row scales linearly with the rows, so the rate in exited tokens/s is the
    whole workload's."""
    import oracle as O
    mask = wl.mask.cpu().numpy()
    ext = wl.ext[: wl.m].cpu().numpy()
    pick = ext[:rows]
    x = wl.h[torch.from_numpy(pick).long().to(wl.h.device)].float().cpu().numpy()
    wk, wv = _w4np(wl.wk), _w4np(wl.wv)
    maps = _host_maps(wl.maps)
    t0 = time.perf_counter()
    O.compact(mask, None)
    O.kv_fill_rows(x, None, len(pick), maps, wk, wv)
    el = time.perf_counter() - t0
    return {"value": len(pick) / el, "unit": "exited tokens/s", "cores": int(_cores()), "kind": "oracle",
            "sample": f"compaction of all {wl.cfg.n_tokens} tokens and the fill of {len(pick)} of the "
                      f"{wl.m} rows through all {wl.nl} layers in "
                      f"{el:.1f} s; the time per row scales linearly with the rows"}


def cpu_baseline_8b(wl):
    """One whole step of the Llama-3-8B prefill on the oracle: route at every
    checkpoint over the running tokens, compaction, the fills at 11 and 31
    (their rows as the GPU step chose them)."""
    import oracle as O
    t_route = t_fill = 0.0
    maps = {c: _host_maps(m) for c, m in wl.maps.items()}
    for c in wl.CKS:
        s = wl.ck[c]
        hp, hc = s["hp"].double().cpu().numpy(), s["hc"].double().cpu().numpy()
        wd, wu = (t.double().cpu().numpy() for t in wl.routers[c])
        t0 = time.perf_counter()
        _, _, mask, _ = O.route(hp, hc, None, 1e-6, wd, wu, -INF, float(np.float32(wl.theta[c])))
        res = O.compact(mask, hc, None if s["ids"] is None else s["ids"].cpu().numpy(), None)
        t_route += time.perf_counter() - t0
        if c in wl.maps:
            wk, wv = (wl.wk1, wl.wv1) if c == wl.e1 else (wl.wk2, wl.wv2)
            t0 = time.perf_counter()
            O.kv_fill_rows(hc, res["exit_idx"], len(res["exit_idx"]), maps[c], _w4np(wk), _w4np(wv))
            t_fill += time.perf_counter() - t0
    el = t_route + t_fill
    return {"value": wl.n / el, "unit": "exited tokens/s", "cores": int(_cores()), "kind": "oracle",
            "route_compact_s": t_route, "fill_s": t_fill,
            "sample": f"one whole step ({wl.n} tokens, 8 checkpoints, fills of "
                      f"{wl.exits[wl.e1]} x 21 and {wl.exits[wl.e2]} x 1 layers) in {el:.1f} s"}


def cpu_baseline_gpt2(wl, target_s):
    """Whole steps of the GPT-2-shape workload on the oracle, repeated for
    about target_s seconds."""
    import oracle as O
    cfg = wl.cfg
    hp = wl.h_prev0.double().cpu().numpy()
    hc = wl.h_cur0.double().cpu().numpy()
    wd = wl.wd.double().cpu().numpy()
    wu = wl.wu.double().cpu().numpy()
    maps = wl.maps.float().cpu().numpy()
    wk, wv = _w4np(wl.wk), _w4np(wl.wv)
    steps, exited = 0, 0
    t0 = time.perf_counter()
    while True:
        _, _, mask, _ = O.route(hp, hc, None, 1e-6, wd, wu, cfg.tau, cfg.theta)
        res = O.compact(mask, hc, None, np.zeros_like(hc))
        ex = res["exit_idx"]
        O.kv_fill_rows(hc, ex, len(ex), maps, wk, wv)
        steps += 1
        exited += len(ex)
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    return {"value": exited / el, "unit": "exited tokens/s", "cores": int(_cores()), "kind": "oracle",
            "sample": f"{steps} whole steps (route of {cfg.n_tokens} tokens, compact, fill of "
                      f"{len(ex)} exited tokens x {wl.nl} layers) in {el:.1f} s"}


def cpu_single_thread_small(gpt2):
    """Single-thread oracle times of the three small workloads: the tiny
    fp32 step (route at block 2, compact, fill of 6 layers through ridge
    maps), one GPT-2-shape step, and the Llama-3.2-1B decode step."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    out = {}
    with threadpool_limits(1):
        # tiny fp32
        cfg = get_config(0)
        e = cfg.route_layers[0]
        hs = G.hidden_states(cfg, cfg.n_tokens, [e - 1, e])
        wd, wu = G.router_weights(cfg, e)
        X, Y = G.calibration(cfg, e)
        maps = O.ridge_fit(X.double().numpy(), Y.double().numpy(), cfg.ridge_lambda)
        w = G.kv_weights(cfg, list(range(e + 1, cfg.L + 1)))
        wk, wv = _w4np(tuple(w["wk"]) + (cfg.group,)), _w4np(tuple(w["wv"]) + (cfg.group,))
        hp, hc = hs[e - 1].double().numpy(), hs[e].double().numpy()
        t0 = time.perf_counter()
        _, _, mask, _ = O.route(hp, hc, None, 1e-6, wd.double().numpy(), wu.double().numpy(), cfg.tau,
                                cfg.theta)
        ex = O.compact(mask, None)["exit_idx"]
        O.kv_fill_rows(hc, ex, len(ex), maps, wk, wv)
        el = time.perf_counter() - t0
        out["tiny fp32 step"] = {"s": el, "exited": int(len(ex)), "exited_tokens_per_s": len(ex) / el}
        # GPT-2 shape
        r = cpu_baseline_gpt2(gpt2, 0.0)
        out["gpt2-small shape step"] = {"exited_tokens_per_s": r["value"], "sample": r["sample"]}
        # Llama-3.2-1B decode step (router off, identity fill)
        dw_cfg = get_config(2)
        n = dw_cfg.n_tokens
        need = sorted({l - 1 for l in dw_cfg.route_layers} | set(dw_cfg.route_layers))
        hs = {l: t.double().numpy() for l, t in G.hidden_states(dw_cfg, n, need).items()}
        w = G.kv_weights(dw_cfg, list(range(1, dw_cfg.L + 1)))
        wk, wv = _w4np(tuple(w["wk"]) + (dw_cfg.group,)), _w4np(tuple(w["wv"]) + (dw_cfg.group,))
        cks = []
        alive = np.ones(n, bool)
        for l in dw_cfg.route_layers:
            cos, _, _, _ = O.route(hs[l - 1], hs[l], None, 1e-6, None, None, -INF, -INF)
            a = np.sort(cos[alive])
            m = len(a)
            tau = float(np.float32(0.5 * (a[(m - 1) // 2] + a[m // 2]))) if m > 1 else -INF
            alive &= ~(cos > tau)
            cks.append({"layer": l, "h_prev": hs[l - 1], "h_cur": hs[l], "tau": tau, "theta": -INF})
        slot = G.slots(dw_cfg).numpy()
        kc = np.zeros((dw_cfg.L, dw_cfg.n_slots, dw_cfg.n_kv_heads, dw_cfg.head_dim))
        t0 = time.perf_counter()
        exl, _, _ = O.decode_step(cks, dw_cfg.L, O.RULE_TOKEN, slot, wk, wv, dw_cfg.n_kv_heads, dw_cfg.head_dim,
                            kc, kc)
        el = time.perf_counter() - t0
        out["llama3.2-1b decode step"] = {"s": el, "us_per_step": el * 1e6,
                                          "filled_token_layers": int(sum(dw_cfg.L - e for e in exl))}
    return out


# ------------------------------------------------------------------ main

def long_context_figures(wl, steps, warmup):
    """The headline: ms per step, exited tokens/s, and the fill split into
    the product of weights and maps (F = deq(W) M per layer) and the
    projection of the rows through F. The fill's own time is a whole-call
    event timing; the two GEMM launches are timed by the library's event
    pairs recorded on the launch stream right around each of them."""
    for i in range(warmup):
        wl.step(i)
    ms_step = time_region(wl.step, steps) / steps
    progress(f"long context N={wl.cfg.n_tokens}: {steps} timed steps, {ms_step:.2f} ms per step")
    reps = max(2, steps // 2)
    tee.river_debug_kernel_times(tee.TIMED_FILL_PROJECTION)     # drop stale records
    tee.river_debug_kernel_times(tee.TIMED_FILL_PRODUCT)
    tee.river_debug_time_kernels(True)
    try:
        fill_ms = time_region(lambda i: wl.fill(i, True), reps) / reps
    finally:
        tee.river_debug_time_kernels(False)
    proj_tot, proj_n = tee.river_debug_kernel_times(tee.TIMED_FILL_PROJECTION)
    prod_tot, prod_n = tee.river_debug_kernel_times(tee.TIMED_FILL_PRODUCT)
    if proj_n != reps or prod_n != reps:
        raise RuntimeError(f"expected {reps} timed projection and product launches, "
                           f"got {proj_n} and {prod_n}")
    proj_ms, prod_ms = proj_tot / proj_n, prod_tot / prod_n
    compact_ms = graph_time(wl.compact, 20)
    map_f, proj_f, prod_f = wl.flops()
    run_f = prod_f + proj_f
    return ms_step, {"fill_ms": fill_ms, "projection_ms": proj_ms, "product_ms": prod_ms,
                     "other_fill_ms": fill_ms - proj_ms - prod_ms,
                     "compact_us": compact_ms * 1e3,
                     "fill_tflops": run_f / (fill_ms * 1e-3) / 1e12,
                     "fill_frac_of_bf16_peak": run_f / (fill_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "product_tflops": prod_f / (prod_ms * 1e-3) / 1e12,
                     "projection_tflops": proj_f / (proj_ms * 1e-3) / 1e12,
                     "product_flops_per_launch": prod_f, "projection_flops_per_launch": proj_f,
                     "two_phase_flops": map_f + proj_f,
                     "note": "fill_tflops counts the flops the fill runs (the product F = deq(W) M per "
                             "layer and the rows through F); the two-phase form (x_hat = M x for every "
                             "row, then its projection) would run two_phase_flops for the same K and V; "
                             "other_fill_ms is the weights' dequantisation and the maps' transposition"}


def long_context_folded_figures(wl, steps, warmup):
    """The long-context step with the 48 maps folded into the K/V weights
    once beforehand (river_kv_fold): compaction, then the rows through F."""
    wl.fold()
    for i in range(warmup):
        wl.step_folded(i)
    ms = time_region(wl.step_folded, steps) / steps
    fill_ms = time_region(wl.fill_folded, max(2, steps // 2)) / max(2, steps // 2)
    _, proj_f, _ = wl.flops()
    out = {"ms_per_step": ms, "exited_tokens_per_s": wl.m / (ms * 1e-3), "fill_ms": fill_ms,
           "fill_tflops": proj_f / (fill_ms * 1e-3) / 1e12,
           "fill_frac_of_bf16_peak": proj_f / (fill_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
           "fold_ms_once": wl.fold_ms,
           "note": "the fill through the folded products F = deq([Wk; Wv]) M of the 48 maps, formed once "
                   "(like the fit) instead of in every step"}
    del wl.F
    torch.cuda.empty_cache()
    return out


def prefill_8b_figures(steps=10, warmup=2, wl=None):
    """The 8B prefill step's figures; wl: an existing workload (e.g. one
    whose fills were folded)."""
    wl = wl or Prefill8BWorkload()
    for i in range(warmup):
        wl.step(i)
    ms = time_region(wl.step, steps) / steps
    rb, cb, ff = wl.work()
    # route and compaction alone over the same checkpoints (every state
    # tensor read once per pass: 1 GB of distinct states per pass)
    def rc(i):
        for c in wl.CKS:
            wl.route(c)
            wl.compact(c)
    rc_ms = time_region(rc, steps) / steps
    fills = {}
    for c in (wl.e1, wl.e2):
        fms = time_region(lambda i: wl.fill(c), steps) / steps
        ne, nl = wl.exits[c], wl.maps[c].shape[0]
        f = wl.fill_flops(c)
        fills[f"exit_at_{c}"] = {"rows": ne, "layers": nl, "ms": fms, "tflops": f / (fms * 1e-3) / 1e12,
                                 "frac_of_bf16_peak": f / (fms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    out = {"workload": "llama3-8b-shape prefill: 8192 tokens, d=4096, 32 blocks, routers (b=128) at "
                       "blocks 3,7,...,31, ~5% exit at 11 (blocks 12-32 filled through 21 ridge maps), "
                       "the rest at 31 (block 32 through one map); states of later checkpoints are the "
                       "continuing tokens'",
           "exits": {str(c): wl.exits[c] for c in wl.CKS if wl.exits[c]},
           "ms_per_step": ms, "exited_tokens_per_s": wl.n / (ms * 1e-3),
           "route_compact_ms": rc_ms, "route_compact_bytes": rb + cb,
           "route_compact_gbs": (rb + cb) / (rc_ms * 1e-3) / 1e9,
           "route_compact_frac_hbm": (rb + cb) / (rc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "fill_flops": ff, "fills": fills, "ridge_fit_ms_22_maps": wl.ridge_ms}
    if getattr(wl, "F", None) is not None:
        out["workload"] += ("; the fills through the folded products F = deq([Wk; Wv]) M of each block's "
                            "map, formed once beforehand")
        out["fold_ms_once"] = wl.fold_ms
    return wl, out


def gpt2_figures(R, steps=200, warmup=20):
    wl = Gpt2Workload(R)
    for i in range(warmup):
        wl.step(i)
    ms = time_region(wl.step, steps) / steps
    n_exit = int(wl.sets[0]["counts"][1].item())
    sets = len(wl.sets)
    k = {}
    for name, fn in (("route", wl.route), ("compact", wl.compact), ("fill", wl.fill),
                     ("projection", wl.fill_projection_only), ("exit_projection", wl.exit_projection),
                     ("fill_layer", wl.fill_layer)):
        k[name] = graph_time(lambda i: fn(wl.sets[i % sets]), max(50, steps // 2), sets)
    rb, cb, ff = wl.work(n_exit)
    cfg = wl.cfg
    ep_bytes = n_exit * (2 * cfg.d * 2 + 4)
    wl.fold()
    for i in range(warmup):
        wl.step_folded(i)
    ms_folded = time_region(wl.step_folded, steps) / steps
    fill_folded = graph_time(lambda i: wl.fill_folded(wl.sets[i % sets]), max(50, steps // 2), sets)
    ff_folded = 2.0 * n_exit * wl.nl * cfg.d * 2 * cfg.n_kv_heads * cfg.head_dim
    folded = {"ms_per_step": ms_folded, "exited_tokens_per_s": n_exit / (ms_folded * 1e-3),
              "fill_us": fill_folded * 1e3, "fill_tflops": ff_folded / (fill_folded * 1e-3) / 1e12,
              "fold_ms_once": wl.fold_ms,
              "note": "the fill through the folded products F = deq([Wk; Wv]) M of the 8 maps, formed once"}
    return wl, {
        "workload": "gpt2-small-shape prefill: 4096 tokens, d=768, L=12, exit check at layer 4 (tau=0.9, "
                    "theta=0.5, router b=128), fill of layers 5-12 through ridge maps and int4 (group 64) "
                    "K/V, 12x64 KV heads",
        "exited_per_step": n_exit, "rotating_sets": sets, "ms_per_step": ms,
        "exited_tokens_per_s": n_exit / (ms * 1e-3),
        "kernel_us": {kk: v * 1e3 for kk, v in k.items()},
        "route_gbs": rb / (k["route"] * 1e-3) / 1e9, "compact_gbs": cb / (k["compact"] * 1e-3) / 1e9,
        "route_compact_frac_hbm": (rb + cb) / ((k["route"] + k["compact"]) * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "fill_tflops": ff / (k["fill"] * 1e-3) / 1e12,
        "exit_projection_gbs": ep_bytes / (k["exit_projection"] * 1e-3) / 1e9,
        "fill_layer_overhead_us": (k["fill_layer"] - k["fill"]) * 1e3,
        "ridge_fit_ms_8_maps": wl.ridge_ms,
        "folded": folded}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only (no sharding across GPUs): --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    tee.load()
    torch.cuda.set_device(0)
    only = args.only
    if only == "copy":
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE calibration
        n = args.copy_probe_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
        return
    if only == "router-fit":
        print(json.dumps({"router_fit": router_fit_all()}))
        return
    if only == "decode3D-folded":
        print(json.dumps({"decode_step_folded": decode_times("3D", 20, folded=True)}))
        return
    if only == "8b-folded":
        wl8 = Prefill8BWorkload()
        wl8.fold()
        _, ff = prefill_8b_figures(args.steps, args.warmup, wl=wl8)
        print(json.dumps({"prefill_8b_folded": ff}))
        return
    if only in ("decode2", "decode3D"):
        key = 2 if only == "decode2" else "3D"
        out = {"decode_step": decode_times(key, 20)}
        if key == "3D":
            out["decode_step_folded"] = decode_times(key, 20, folded=True)
        print(json.dumps(out))
        return
    if only == "route-compact":
        print(json.dumps({"route_compact_8b_cold": route_compact_8b_cold()}))
        return
    if only == "8b":
        wl8, f = prefill_8b_figures(args.steps, args.warmup)
        wl8.fold()
        _, ff = prefill_8b_figures(args.steps, args.warmup, wl=wl8)
        print(json.dumps({"prefill_8b": f, "prefill_8b_folded": ff}))
        return
    if only == "gpt2":
        _, f = gpt2_figures(args.rotate, max(args.steps, 50), args.warmup)
        print(json.dumps({"gpt2": f}))
        return

    # ---- the headline: long-context prefill
    wl = LongContextWorkload(args.tokens)
    progress(f"long context N={args.tokens}: {wl.m} rows x {wl.nl} layers, maps fitted in "
             f"{wl.ridge_ms:.0f} ms")
    ms_step, lc = long_context_figures(wl, args.steps, args.warmup)
    lcf = long_context_folded_figures(wl, args.steps, args.warmup)
    if only == "long":
        print(json.dumps({"long_context": lc, "ms_per_step": ms_step, "long_context_folded": lcf}))
        return
    value = wl.m / (ms_step * 1e-3)
    ach = lc["projection_flops_per_launch"] / (lc["projection_ms"] * 1e-3) / 1e12
    roof = {"kernel": "gemm_quad_kernel<2> (the projection: [K|V] = X F^T into the cache for all 48 "
                      "layers in one launch)",
            "bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / MFMA_BF16_PEAK_TFLOPS,
            "traffic": measured_traffic(f"projection_long_context_{args.tokens}_traffic.json",
                                        GEMM_SOURCES),
            "flops_per_launch": lc["projection_flops_per_launch"], "avg_launch_ms": lc["projection_ms"],
            "duration_method": "HIP events recorded by the library on the launch stream right before "
                               "and after each projection launch of the timed fills, averaged"}
    cfg = wl.cfg
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
        "config": {"workload": f"ridgefill long-context prefill: N={cfg.n_tokens} tokens, d=5120, 64 blocks, "
                               f"split after block 16, rows 16..N-2048 ({wl.m}) exit (positional rule, "
                               f"compacted) and fill blocks 17-64 through 48 ridge maps fitted on the GPU "
                               f"from {wl.n_calib} calibration tokens (lambda=0.1), int4 (group 128) K/V, "
                               f"8x128 KV heads, Student-t (nu=5) states; the fill forms per layer the "
                               f"product of the dequantised K/V weights and the map and projects the rows "
                               f"through it",
                   "exited_per_step": wl.m, "layers_filled": wl.nl},
        "fill_tflops": lc["fill_tflops"],
        "fill_frac_of_bf16_peak": lc["fill_frac_of_bf16_peak"],
        "long_context": lc,
        "long_context_folded": lcf,
        "ridge_fit_ms_48_maps": wl.ridge_ms,
        "roofline": roof,
    }
    cpu = None
    if not args.no_cpu_baseline:
        model, blas = host_info()
        cpu = cpu_baseline_long(wl)
        cpu["cpu_model"], cpu["blas"] = model, blas
        progress("cpu baseline (long context) done")
    del wl
    torch.cuda.empty_cache()

    wl8, line["prefill_8b"] = prefill_8b_figures()
    wl8.fold()
    _, line["prefill_8b_folded"] = prefill_8b_figures(wl=wl8)
    progress("8B prefill step done")
    line["route_compact_8b_cold"] = route_compact_8b_cold()
    progress("8B route and compaction (cold) done")
    wl1, line["gpt2_prefill"] = gpt2_figures(args.rotate)
    progress("GPT-2-shape step done")
    line["decode_step"] = {
        "llama3.2-1b decode: 64 tokens, d=2048, checks after blocks 8..15 (router off), identity fill":
            decode_times(2, 50),
        "llama3-8b decode: 256 tokens, d=4096, 8 router checkpoints, maps for the exits at 11 and 31":
            decode_times("3D", 20),
        "llama3-8b decode, maps folded into the K/V weights beforehand":
            decode_times("3D", 20, folded=True),
    }
    progress("decode steps done")
    line["router_fit"] = router_fit_all()
    progress("router calibration done")
    if cpu is not None:
        cpu["by_workload"] = {"llama3-8b prefill step": cpu_baseline_8b(wl8),
                              "gpt2-small prefill steps": cpu_baseline_gpt2(wl1, 5.0),
                              "single thread": cpu_single_thread_small(wl1)}
        line["cpu_baseline"] = cpu
        progress("cpu baselines done")
    print(json.dumps(line))


if __name__ == "__main__":
    main()
