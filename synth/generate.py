"""Seeded input generators (torch, on CPU for small workloads, on the GPU
for the large ones).

Recipe (one stream per named tensor, seeded from (config, name), so a
tensor does not change when another one is added or dropped):

* hidden states: h^(0) ~ N(0, I); h^(l) = h^(l-1) + sigma_l * eps_l with
  eps ~ N(0, I) and sigma_l = 0.5 * 0.7**l, so the cosine between a block's
  input and output rises with depth (River-LLM, "核心方法", Fig. 6b).
  The long-context case draws h^(0) and eps from Student-t with nu = 5
  scaled by sqrt(3/5) to unit variance. The Llama-3.2-1B decode case uses
  a per-token, per-layer step sigma ~ U(0.05, 0.5) from layer 8 on, which
  spreads the cosines so that a per-layer threshold splits the batch.
  States are accumulated in fp32 and each stored layer is rounded to the
  workload dtype.
* router: W_down ~ N(0, 1/d), W_up ~ N(0, 1/b), gamma = 1 (passed as NULL).
* final RMSNorm weight (exit projection): gamma = 1 + 0.1 * N(0, 1), the
  spread of a trained norm's weights around one.
* the skipped layers' own K/V path: input RMSNorm weights gamma_l = 1 +
  0.1 * N(0, 1) per layer, K/V biases N(0, 0.02^2), rotary tables
  cos/sin(p * base^(-2i/head_dim)) in fp32 (computed in float64), base
  500000 for the Llama-3-shape workloads and 10000 otherwise.
* K/V weights: W ~ N(0, 1/d) per layer, stored as int4 with a per-group
  scale and zero (round-to-nearest, min-max; see ``quantize_w4``).
* decode slots: distinct, drawn without replacement; prefill slots are the
  token positions.
* router calibration states (one checkpoint): h_k from the calibration
  walk; the drift to the final layer is s_i * |h_k| / sqrt(d) * N(0, I) with
  s_i = 0.25 * exp(-q_i), q_i = sqrt(d) * <h_k / |h_k|, v> for a fixed unit
  direction v. About 40% of the tokens then end within cosine 0.98 of
  their final state, and which ones is learnable from h_k alone.
"""

import math
import zlib

import torch

from .configs import Config, sigma

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name):
    return _DT[name]


def stream(cfg_idx, name, device="cpu"):
    """torch.Generator for one named tensor of one workload (seed 0)."""
    # seed 0 of the workload, mixed with the workload id and the tensor name
    seed = ((hash_cfg(cfg_idx) << 32) ^ zlib.crc32(name.encode())) & ((1 << 63) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def hash_cfg(cfg_idx):
    return zlib.crc32(str(cfg_idx).encode()) & 0x7FFFFFFF


def _normal(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _student_t5(shape, gen, device):
    """Student-t with 5 degrees of freedom, scaled to unit variance:
    t = z0 / sqrt(sum_{i=1..5} z_i^2 / 5), times sqrt(3/5)."""
    z0 = _normal(shape, gen, device)
    chi = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(5):
        zi = _normal(shape, gen, device)
        chi += zi * zi
    return z0 / torch.sqrt(chi / 5.0) * math.sqrt(3.0 / 5.0)


def _draw(cfg, shape, gen, device):
    return _student_t5(shape, gen, device) if cfg.student_t else _normal(shape, gen, device)


def hidden_states(cfg: Config, n, layers, tag="eval", device="cpu", dtype=None):
    """States h^(l) for the requested layers of n tokens.

    Returns {l: tensor [n][d]} in the workload dtype (or ``dtype``).
    ``tag`` separates the evaluated tokens from the calibration tokens.
    """
    dt = _DT[cfg.dtype] if dtype is None else dtype
    want = sorted(set(int(l) for l in layers))
    top = want[-1]
    gen = stream(cfg.idx, f"h/{tag}", device)
    h = _draw(cfg, (n, cfg.d), gen, device)
    out = {}
    if 0 in want:
        out[0] = h.to(dt)
    spread = cfg.idx == 2  # decode case: per-token step sizes from L_s on
    for l in range(1, top + 1):
        eps = _draw(cfg, (n, cfg.d), gen, device)
        if spread and l >= 8:
            s = torch.rand((n, 1), generator=gen, device=device) * 0.45 + 0.05
            h = h + s * eps
        else:
            h = h + sigma(l) * eps
        if l in want:
            out[l] = h.to(dt)
    return out


def router_weights(cfg: Config, layer, device="cpu"):
    """(W_down [b][d], W_up [b]) of the router at checkpoint ``layer``."""
    dt = _DT[cfg.dtype]
    g = stream(cfg.idx, f"router/{layer}", device)
    w_down = _normal((cfg.b, cfg.d), g, device) / math.sqrt(cfg.d)
    w_up = _normal((cfg.b,), g, device) / math.sqrt(cfg.b)
    return w_down.to(dt), w_up.to(dt)


def final_norm_gamma(cfg: Config, device="cpu"):
    """Weight [d] of the final RMSNorm, in the workload dtype."""
    g = stream(cfg.idx, "final_norm", device)
    return (1.0 + 0.1 * _normal((cfg.d,), g, device)).to(_DT[cfg.dtype])


def layer_norm_gammas(cfg: Config, layers, device="cpu"):
    """Input RMSNorm weights [len(layers)][d] of the given layers."""
    out = []
    for l in layers:
        g = stream(cfg.idx, f"layer_norm/{l}", device)
        out.append(1.0 + 0.1 * _normal((cfg.d,), g, device))
    return torch.stack(out).to(_DT[cfg.dtype]).contiguous()


def kv_biases(cfg: Config, layers, device="cpu"):
    """(K bias, V bias), each [len(layers)][n_kv_heads * head_dim]."""
    n_out = cfg.n_kv_heads * cfg.head_dim
    res = []
    for which in ("k", "v"):
        out = []
        for l in layers:
            g = stream(cfg.idx, f"bias/{which}/{l}", device)
            out.append(0.02 * _normal((n_out,), g, device))
        res.append(torch.stack(out).to(_DT[cfg.dtype]).contiguous())
    return tuple(res)


def rope_base(cfg: Config):
    return 500000.0 if cfg.idx in (2, 3) else 10000.0


def rope_tables(cfg: Config, n_pos, device="cpu"):
    """(cos, sin), each fp32 [n_pos][head_dim / 2]."""
    hd = cfg.head_dim
    inv = rope_base(cfg) ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = torch.arange(n_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return (torch.cos(ang).float().contiguous().to(device),
            torch.sin(ang).float().contiguous().to(device))


def quantize_w4(w, group, sz_dtype):
    """Round-to-nearest asymmetric int4 storage of fp32 weights.

    Per output row and per group of ``group`` input channels:
    scale = (max - min) / 15 (1 when max == min), zero = -min / scale, both
    stored in ``sz_dtype``; q = clip(round(w / scale + zero), 0, 15) with the
    stored scale and zero. Packing: element k in byte k // 2, low nibble when
    k is even.

    w: [..., n_out, k] float32. Returns (q uint8 [..., n_out, k/2],
    scale, zero [..., n_out, k/group]).
    """
    dt = _DT[sz_dtype]
    *lead, n_out, k = w.shape
    wg = w.reshape(*lead, n_out, k // group, group)
    mn = wg.amin(dim=-1)
    mx = wg.amax(dim=-1)
    s = (mx - mn) / 15.0
    s = torch.where(s == 0, torch.ones_like(s), s)
    z = -mn / s
    s_st = s.to(dt)
    z_st = z.to(dt)
    sf = s_st.float().unsqueeze(-1)
    zf = z_st.float().unsqueeze(-1)
    q = torch.clamp(torch.round(wg / sf + zf), 0, 15).to(torch.uint8)
    q = q.reshape(*lead, n_out, k)
    packed = (q[..., 0::2] | (q[..., 1::2] << 4)).contiguous()
    return packed, s_st.contiguous(), z_st.contiguous()


def kv_weights(cfg: Config, layers, device="cpu"):
    """int4 K and V projections of the given layers, stacked in order.

    Returns dict(wk=(q, s, z), wv=(q, s, z)) with q [n][hd][d/2] and s, z
    [n][hd][d/group].
    """
    qs = {"k": ([], [], []), "v": ([], [], [])}
    for l in layers:
        for which in ("k", "v"):
            g = stream(cfg.idx, f"w{which}/{l}", device)
            w = _normal((cfg.hd, cfg.d), g, device) / math.sqrt(cfg.d)
            q, s, z = quantize_w4(w, cfg.group, cfg.sz_dtype)
            qs[which][0].append(q)
            qs[which][1].append(s)
            qs[which][2].append(z)
    res = {}
    for which in ("k", "v"):
        res["w" + which] = tuple(torch.stack(x).contiguous() for x in qs[which])
    return res


def router_calibration(cfg: Config, k, n=None, device="cpu"):
    """(h_k, h_final), each [n][d] in the workload dtype, for training the
    router at checkpoint k."""
    n = cfg.n_calib if n is None else n
    hk = hidden_states(cfg, n, [k], tag="router_calib", device=device, dtype=torch.float32)[k]
    g = stream(cfg.idx, f"router_calib/{k}", device)
    v = _normal((cfg.d,), g, device)
    v = v / v.norm()
    nrm = hk.norm(dim=1, keepdim=True)
    q = (hk @ v)[:, None] / nrm * math.sqrt(cfg.d)
    s = 0.25 * torch.exp(-q)
    drift = _normal((n, cfg.d), g, device)
    hf = hk + s * drift * nrm / math.sqrt(cfg.d)
    dt = _DT[cfg.dtype]
    return hk.to(dt).contiguous(), hf.to(dt).contiguous()


def slots(cfg: Config, n=None, device="cpu"):
    """Cache slot of each evaluated token (int32)."""
    n = cfg.n_tokens if n is None else n
    if not cfg.decode:
        return torch.arange(n, dtype=torch.int32, device=device)
    g = stream(cfg.idx, "slots", "cpu")
    perm = torch.randperm(cfg.n_slots - cfg.slot_lo, generator=g)[:n] + cfg.slot_lo
    return perm.to(torch.int32).to(device)


def calibration(cfg: Config, e, n=None, device="cpu"):
    """Ridge calibration pairs for exit layer e: X = h^(e) of the
    calibration tokens and Y[l - e - 1] = h^(l-1), the input of block l,
    for l = e+1..L. Returns (X [n][d], Y [L-e][n][d])."""
    n = cfg.n_calib if n is None else n
    layers = list(range(e, cfg.L))
    hs = hidden_states(cfg, n, layers, tag="calib", device=device)
    X = hs[e]
    Y = torch.stack([hs[l] for l in layers])
    return X, Y


def near_identity_maps(cfg: Config, n_maps, scale=0.05, tag="maps", device="cpu"):
    """Stand-in maps I + N(0, scale^2/d) in the workload dtype, output-major,
    for fill tests whose map values need not come from a fit."""
    g = stream(cfg.idx, tag, device)
    m = _normal((n_maps, cfg.d, cfg.d), g, device) * (scale / math.sqrt(cfg.d))
    m += torch.eye(cfg.d, device=device)
    return m.to(_DT[cfg.dtype])


def nan_cache(cfg: Config, n_layers, device="cpu"):
    """K and V caches filled with a NaN sentinel."""
    shape = (n_layers, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim)
    dt = _DT[cfg.dtype]
    return (torch.full(shape, float("nan"), dtype=dt, device=device),
            torch.full(shape, float("nan"), dtype=dt, device=device))
