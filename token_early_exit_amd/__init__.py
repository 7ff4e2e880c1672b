"""Python binding of libriver (the per-token exit-and-KV-fill library).

Argument marshalling only: every function forwards torch tensors' device
pointers and the current HIP stream to the C interface declared in
``include/river.h``; all arithmetic runs in the HIP kernels. There is no
CPU fallback: if the library is not built, ``load()`` raises.

The calls keep the C names: ``river_route``, ``river_compact``,
``river_exit_projection``, ``river_kv_fill``, ``river_kv_fill_layer``,
``river_decode_step``, ``river_decode_step_static``, ``river_router_fit``,
``river_ridge_fit``; plus ``river_workspace_size``.
"""

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libriver.so")

RIVER_F32, RIVER_BF16 = 0, 1
RULE_TOKEN, RULE_BATCH_MIN = 0, 1
TIMED_FILL_PROJECTION, TIMED_FILL_PRODUCT = 0, 1
(OP_ROUTE, OP_COMPACT, OP_KV_FILL, OP_RIDGE_FIT, OP_KV_FILL_LAYER, OP_DECODE_STEP,
 OP_ROUTER_FIT, OP_KV_FOLD) = 0, 1, 2, 3, 4, 5, 6, 7
STATUS = {0: "OK", 1: "ERR_ARG", 2: "ERR_DTYPE", 3: "ERR_ALIGN", 4: "ERR_UNSUPPORTED",
          5: "ERR_WORKSPACE", 6: "ERR_NOT_SPD", 7: "ERR_HIP"}

EXPORTS = ["river_route", "river_compact", "river_exit_projection", "river_kv_fill",
           "river_kv_fill_layer", "river_kv_fold", "river_kv_fill_folded", "river_decode_step", "river_router_fit", "river_ridge_fit",
           "river_workspace_size", "river_last_error", "river_version",
           "river_debug_set_compact_path", "river_debug_set_gemm_path",
           "river_debug_set_decode_path", "river_debug_set_fill_fuse", "river_debug_kv_fill_plan", "river_decode_step_static",
           "river_debug_time_kernels", "river_debug_kernel_times"]


class RiverError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class RiverW4(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("zero", ctypes.c_void_p),
                ("sz_dtype", ctypes.c_int), ("group", ctypes.c_int)]


class RiverLayer(ctypes.Structure):
    _fields_ = [("norm_gamma", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("k_bias", ctypes.c_void_p), ("v_bias", ctypes.c_void_p),
                ("pos", ctypes.c_void_p), ("rope_cos", ctypes.c_void_p),
                ("rope_sin", ctypes.c_void_p), ("n_pos", ctypes.c_int64)]


class RiverCheckpoint(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int), ("h_prev", ctypes.c_void_p), ("h_cur", ctypes.c_void_p),
                ("tau", ctypes.c_float), ("theta", ctypes.c_float), ("w_down", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("maps", ctypes.c_void_p), ("folded", ctypes.c_void_p)]


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_F = ctypes.c_float
_S = ctypes.c_size_t


def load():
    """Load libriver.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    lib.river_route.argtypes = [_I, _I, _I, _P, _L, _P, _L, _P, _F, _P, _P, _I, _F, _F, _I,
                                _P, _P, _P, _P, _P]
    lib.river_compact.argtypes = [_I, _I, _I, _P, _P, _L, _P, _P, _P, _P, _P, _L, _P, _P, _L, _L,
                                  _P, _S, _P]
    lib.river_exit_projection.argtypes = [_I, _P, _I, _I, _P, _L, _I, _P, _P, _P, _F, _P, _L, _L,
                                          _P]
    lib.river_kv_fill.argtypes = [_I, _P, _I, _I, _P, _L, _I, _P, _P, _I, _P,
                                  ctypes.POINTER(RiverW4), ctypes.POINTER(RiverW4), _I, _I,
                                  _P, _P, _L, _P, _S, _P]
    lib.river_kv_fill_layer.argtypes = [_I, _P, _I, _I, _P, _L, _I, _P, _P, _I, _P,
                                        ctypes.POINTER(RiverW4), ctypes.POINTER(RiverW4),
                                        ctypes.POINTER(RiverLayer), _I, _I, _P, _P, _L, _P, _S, _P]
    lib.river_decode_step.argtypes = [_I, _I, _I, _L, _I, ctypes.POINTER(RiverCheckpoint), _I, _P, _F,
                                      _I, _I, ctypes.POINTER(RiverW4), ctypes.POINTER(RiverW4), _I,
                                      _I, _P, _P, _P, _L, _P, _P, _S, _P]
    lib.river_decode_step_static.argtypes = [_I, _I, _I, _L, _I, ctypes.POINTER(RiverCheckpoint), _I, _P,
                                             _F, _I, _I, ctypes.POINTER(RiverW4),
                                             ctypes.POINTER(RiverW4), _I, _I, _P, _P, _P, _L, _P, _P]
    lib.river_kv_fold.argtypes = [_I, _I, _P, ctypes.POINTER(RiverW4), ctypes.POINTER(RiverW4), _I, _I, _P,
                                  _P, _S, _P]
    lib.river_kv_fill_folded.argtypes = [_I, _P, _I, _P, _L, _I, _P, _P, _I, _P, _I, _I, _P, _P, _L, _P]
    lib.river_router_fit.argtypes = [_I, _I, _I, _P, _L, _P, _P, _F, _I, _P, _P, _I, _I, _P, _F, _F,
                                     _F, _F, _P, _P, _S, _P]
    lib.river_ridge_fit.argtypes = [_I, _I, _I, _I, _P, _I, _P, _I, _F, _P, _I, _P, _S, _P]
    for f in ("river_route", "river_compact", "river_exit_projection", "river_kv_fill",
              "river_kv_fill_layer", "river_kv_fold", "river_kv_fill_folded",
              "river_decode_step", "river_decode_step_static",
              "river_router_fit", "river_ridge_fit",
              "river_debug_set_compact_path", "river_debug_set_gemm_path", "river_debug_set_decode_path",
              "river_debug_set_fill_fuse", "river_debug_time_kernels", "river_debug_kernel_times"):
        getattr(lib, f).restype = _I
    lib.river_debug_set_compact_path.argtypes = [_I]
    lib.river_debug_set_gemm_path.argtypes = [_I]
    lib.river_debug_set_decode_path.argtypes = [_I]
    lib.river_debug_set_fill_fuse.argtypes = [_I]
    lib.river_debug_time_kernels.argtypes = [_I]
    lib.river_debug_kernel_times.argtypes = [_I, _P, _P]
    lib.river_debug_kv_fill_plan.argtypes = [_I, _I, _I, _I, _I, _S, _P, _P, _P]
    lib.river_debug_kv_fill_plan.restype = _I
    lib.river_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I]
    lib.river_workspace_size.restype = _S
    lib.river_last_error.restype = ctypes.c_char_p
    lib.river_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ----------------------------------------------------------- marshalling

def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dt(t):
    import torch
    if t.dtype == torch.bfloat16:
        return RIVER_BF16
    if t.dtype == torch.float32:
        return RIVER_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(st):
    if st != 0:
        raise RiverError(st, load().river_last_error().decode())


def _ld(t):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("matrices must be 2-D with unit column stride")
    return t.stride(0)


def version():
    return load().river_version().decode()


def river_workspace_size(op, n=0, d=0, d_out=0, n_targets=0, n_layers=0):
    return load().river_workspace_size(op, n, d, d_out, n_targets, n_layers)


def river_debug_set_compact_path(path):
    _check(load().river_debug_set_compact_path(path))


def river_debug_set_gemm_path(path):
    _check(load().river_debug_set_gemm_path(path))


def river_debug_set_decode_path(path):
    _check(load().river_debug_set_decode_path(path))


def river_debug_set_fill_fuse(mode):
    _check(load().river_debug_set_fill_fuse(mode))


def river_debug_time_kernels(on):
    _check(load().river_debug_time_kernels(int(bool(on))))


def river_debug_kernel_times(kind):
    """(total ms, launches) of the recorded launches of one kind
    (TIMED_FILL_PROJECTION or TIMED_FILL_PRODUCT); clears them."""
    ms, n = ctypes.c_double(), ctypes.c_int()
    _check(load().river_debug_kernel_times(kind, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def river_debug_kv_fill_plan(m_max, d, n_out, n_layers, ws_bytes, dev_count=False):
    """(layers per chunk, projection path, parts) of a plain bf16 fill with
    maps; path 0 = int4 in registers, 1 = split reduction, 2 = dequantised
    weights, 3 = through the product of the weights and the maps."""
    c, p, k = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(load().river_debug_kv_fill_plan(m_max, int(bool(dev_count)), d, n_out, n_layers, ws_bytes,
                                           ctypes.byref(c), ctypes.byref(p), ctypes.byref(k)))
    return c.value, p.value, k.value


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_w4(w, n_layers, n_out, d, name):
    q, s, z, group = w
    _need(q.dim() == 3 and tuple(q.shape) == (n_layers, n_out, d // 2),
          f"{name}: q must be [{n_layers}][{n_out}][{d // 2}], got {tuple(q.shape)}")
    _need(group > 0 and d % group == 0, f"{name}: group {group} must divide d = {d}")
    for t, nm in ((s, "scale"), (z, "zero")):
        _need(tuple(t.shape) == (n_layers, n_out, d // group),
              f"{name}: {nm} must be [{n_layers}][{n_out}][{d // group}], got {tuple(t.shape)}")


def _check_fill(h, slot, wk, wv, n_kv_heads, head_dim, k_cache, v_cache, m_max, m_dev, row_idx,
                maps, n_layers):
    """Shapes a fill reads and writes, checked against each other (the C
    interface takes bare pointers and cannot): a mismatch raises here
    instead of becoming an out-of-bounds device access."""
    n_rows, d = h.shape
    n_out = n_kv_heads * head_dim
    _check_w4(wk, n_layers, n_out, d, "wk")
    _check_w4(wv, n_layers, n_out, d, "wv")
    for c, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(c.dim() == 4 and c.shape[0] == n_layers and tuple(c.shape[2:]) == (n_kv_heads, head_dim),
              f"{nm} must be [{n_layers}][n_slots][{n_kv_heads}][{head_dim}], got {tuple(c.shape)}")
        _need(c.is_contiguous(), f"{nm} must be contiguous")
    _need(k_cache.shape[1] == v_cache.shape[1], "k_cache and v_cache must have the same slot count")
    _need(slot.dim() == 1 and slot.shape[0] >= n_rows,
          f"slot must hold one entry per row of h ({n_rows}), got {tuple(slot.shape)}")
    if row_idx is not None:
        _need(row_idx.dim() == 1 and row_idx.shape[0] >= m_max,
              f"row_idx must hold m_max = {m_max} entries, got {tuple(row_idx.shape)}")
    if m_dev is not None:
        _need(m_dev.numel() >= 1, "m_dev must hold one count")
    if maps is not None:
        _need(tuple(maps.shape) == (n_layers, d, d) and maps.is_contiguous(),
              f"maps must be contiguous [{n_layers}][{d}][{d}], got {tuple(maps.shape)}")


def river_route(h_prev, h_cur, mask_out, *, gamma=None, eps=1e-6, w_down=None, w_up=None,
                tau=-math.inf, theta=-math.inf, rule=RULE_TOKEN, cos_out=None, prob_out=None,
                all_exit_out=None, stream=None):
    n, d = h_cur.shape
    b = 0 if w_down is None else w_down.shape[0]
    _need(tuple(h_prev.shape) == (n, d), f"h_prev must be [{n}][{d}] like h_cur, got {tuple(h_prev.shape)}")
    _need(mask_out.numel() >= n, f"mask_out must hold {n} entries")
    for t, nm in ((cos_out, "cos_out"), (prob_out, "prob_out")):
        if t is not None:
            _need(t.numel() >= n, f"{nm} must hold {n} entries")
    if gamma is not None:
        _need(gamma.numel() == d, f"gamma must hold d = {d} entries")
    if w_down is not None:
        _need(w_down.dim() == 2 and w_down.shape[1] == d and w_down.is_contiguous(),
              f"w_down must be contiguous [b][{d}]")
        _need(w_up is not None and w_up.numel() == b, f"w_up must hold b = {b} entries")
    _check(load().river_route(n, d, _dt(h_cur), _ptr(h_prev), _ld(h_prev), _ptr(h_cur), _ld(h_cur),
                              _ptr(gamma), eps, _ptr(w_down), _ptr(w_up), b, tau, theta, rule,
                              _ptr(cos_out), _ptr(prob_out), _ptr(mask_out), _ptr(all_exit_out),
                              _stream(stream)))


def river_compact(mask, h, cont_idx, exit_idx, counts, *, row_ids=None, h_cont=None,
                  row_ids_cont=None, out=None, workspace=None, stream=None, d=None, dt=None):
    n = mask.shape[0]
    if h is not None:
        d, dt = h.shape[1], _dt(h)
        ld_h = _ld(h)
    else:
        ld_h = 0
        d = d or 8
        dt = RIVER_BF16 if dt is None else dt
    for t, nm in ((cont_idx, "cont_idx"), (exit_idx, "exit_idx")):
        _need(t.numel() >= n, f"{nm} must hold {n} entries")
    _need(counts.numel() >= 2, "counts must hold 2 entries")
    if h is not None:
        _need(h.shape[0] >= n, f"h must hold {n} rows")
    if row_ids is not None:
        _need(row_ids.numel() >= n, f"row_ids must hold {n} entries")
    if h_cont is not None:
        _need(h_cont.shape[0] >= n and h_cont.shape[1] == d, f"h_cont must be [{n}][{d}]")
    if row_ids_cont is not None:
        _need(row_ids_cont.numel() >= n, f"row_ids_cont must hold {n} entries")
    if out is not None:
        _need(out.shape[1] == d, f"out must have d = {d} columns")
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().river_compact(n, d, dt, _ptr(mask), _ptr(h), ld_h, _ptr(row_ids), _ptr(cont_idx),
                                _ptr(exit_idx), _ptr(counts), _ptr(h_cont),
                                _ld(h_cont) if h_cont is not None else 0, _ptr(row_ids_cont),
                                _ptr(out), _ld(out) if out is not None else 0,
                                out.shape[0] if out is not None else 0, _ptr(workspace), ws_n,
                                _stream(stream)))


def river_exit_projection(h, out, *, m_max=None, m_dev=None, row_idx=None, row_ids=None,
                          gamma=None, eps=1e-6, stream=None):
    n_rows, d = h.shape
    if m_max is None:
        m_max = row_idx.shape[0] if row_idx is not None else n_rows
    _need(out.dim() == 2 and out.shape[1] == d, f"out must have d = {d} columns")
    if row_idx is not None:
        _need(row_idx.numel() >= m_max, f"row_idx must hold m_max = {m_max} entries")
    if row_ids is not None:
        _need(row_ids.numel() >= n_rows, f"row_ids must hold one entry per row of h ({n_rows})")
    if gamma is not None:
        _need(gamma.numel() == d, f"gamma must hold d = {d} entries")
    _check(load().river_exit_projection(m_max, _ptr(m_dev), d, _dt(h), _ptr(h), _ld(h), n_rows,
                                        _ptr(row_idx), _ptr(row_ids), _ptr(gamma), eps, _ptr(out),
                                        _ld(out), out.shape[0], _stream(stream)))


def w4(q, scale, zero, group):
    """int4 descriptor from (q, scale, zero) tensors; keeps no reference."""
    return RiverW4(q.data_ptr(), scale.data_ptr(), zero.data_ptr(), _dt(scale), group)


def river_kv_fill(h, slot, wk, wv, n_kv_heads, head_dim, k_cache, v_cache, *, m_max=None,
                  m_dev=None, row_idx=None, maps=None, workspace=None, stream=None):
    """wk, wv: (q, scale, zero, group) tuples of tensors."""
    n_rows, d = h.shape
    n_layers = wk[0].shape[0]
    if m_max is None:
        m_max = row_idx.shape[0] if row_idx is not None else n_rows
    _check_fill(h, slot, wk, wv, n_kv_heads, head_dim, k_cache, v_cache, m_max, m_dev, row_idx,
                maps, n_layers)
    dk = w4(*wk)
    dv = w4(*wv)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().river_kv_fill(m_max, _ptr(m_dev), d, _dt(h), _ptr(h), _ld(h), n_rows,
                                _ptr(row_idx), _ptr(slot), n_layers, _ptr(maps),
                                ctypes.byref(dk), ctypes.byref(dv), n_kv_heads, head_dim,
                                _ptr(k_cache), _ptr(v_cache), k_cache.shape[1], _ptr(workspace),
                                ws_n, _stream(stream)))


def river_kv_fold(wk, wv, n_kv_heads, head_dim, F, *, maps=None, workspace=None, stream=None):
    """F[l] = deq([Wk[l]; Wv[l]]) . maps[l] (bf16 [n_layers][2 n_out][d]);
    wk, wv: (q, scale, zero, group) tuples; maps None folds the identity."""
    n_layers, n_out, half = wk[0].shape
    d = 2 * half
    _check_w4(wk, n_layers, n_out, d, "wk")
    _check_w4(wv, n_layers, n_out, d, "wv")
    _need(n_out == n_kv_heads * head_dim, f"wk holds {n_out} outputs, not n_kv_heads * head_dim")
    _need(tuple(F.shape) == (n_layers, 2 * n_out, d) and F.is_contiguous() and _dt(F) == RIVER_BF16,
          f"F must be contiguous bf16 [{n_layers}][{2 * n_out}][{d}], got {tuple(F.shape)}")
    if maps is not None:
        _need(tuple(maps.shape) == (n_layers, d, d) and maps.is_contiguous() and _dt(maps) == RIVER_BF16,
              f"maps must be contiguous bf16 [{n_layers}][{d}][{d}], got {tuple(maps.shape)}")
    dk = w4(*wk)
    dv = w4(*wv)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().river_kv_fold(d, n_layers, _ptr(maps), ctypes.byref(dk), ctypes.byref(dv), n_kv_heads,
                                head_dim, _ptr(F), _ptr(workspace), ws_n, _stream(stream)))


def river_kv_fill_folded(h, slot, F, n_kv_heads, head_dim, k_cache, v_cache, *, m_max=None, m_dev=None,
                         row_idx=None, stream=None):
    """river_kv_fill through F from river_kv_fold (bf16 throughout)."""
    n_rows, d = h.shape
    n_layers = F.shape[0]
    n_out = n_kv_heads * head_dim
    if m_max is None:
        m_max = row_idx.shape[0] if row_idx is not None else n_rows
    _need(tuple(F.shape) == (n_layers, 2 * n_out, d) and F.is_contiguous() and _dt(F) == RIVER_BF16,
          f"F must be contiguous bf16 [{n_layers}][{2 * n_out}][{d}], got {tuple(F.shape)}")
    _need(_dt(h) == RIVER_BF16 and _dt(k_cache) == RIVER_BF16 and _dt(v_cache) == RIVER_BF16,
          "the folded fill takes bf16 states and caches")
    for c, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(c.dim() == 4 and c.shape[0] == n_layers and tuple(c.shape[2:]) == (n_kv_heads, head_dim),
              f"{nm} must be [{n_layers}][n_slots][{n_kv_heads}][{head_dim}], got {tuple(c.shape)}")
        _need(c.is_contiguous(), f"{nm} must be contiguous")
    _need(k_cache.shape[1] == v_cache.shape[1], "k_cache and v_cache must have the same slot count")
    _need(slot.dim() == 1 and slot.shape[0] >= n_rows,
          f"slot must hold one entry per row of h ({n_rows}), got {tuple(slot.shape)}")
    if row_idx is not None:
        _need(row_idx.dim() == 1 and row_idx.shape[0] >= m_max,
              f"row_idx must hold m_max = {m_max} entries, got {tuple(row_idx.shape)}")
    if m_dev is not None:
        _need(m_dev.numel() >= 1, "m_dev must hold one count")
    _check(load().river_kv_fill_folded(m_max, _ptr(m_dev), d, _ptr(h), _ld(h), n_rows, _ptr(row_idx),
                                       _ptr(slot), n_layers, _ptr(F), n_kv_heads, head_dim, _ptr(k_cache),
                                       _ptr(v_cache), k_cache.shape[1], _stream(stream)))


def river_kv_fill_layer(h, slot, wk, wv, n_kv_heads, head_dim, k_cache, v_cache, *, m_max=None,
                        m_dev=None, row_idx=None, maps=None, norm_gamma=None, norm_eps=1e-6,
                        k_bias=None, v_bias=None, pos=None, rope_cos=None, rope_sin=None,
                        workspace=None, stream=None):
    """river_kv_fill through the layer's input RMSNorm, K/V bias and the
    rotary embedding of K (each off when its tensor is None)."""
    n_rows, d = h.shape
    n_layers = wk[0].shape[0]
    if m_max is None:
        m_max = row_idx.shape[0] if row_idx is not None else n_rows
    _check_fill(h, slot, wk, wv, n_kv_heads, head_dim, k_cache, v_cache, m_max, m_dev, row_idx,
                maps, n_layers)
    n_out = n_kv_heads * head_dim
    if norm_gamma is not None:
        _need(tuple(norm_gamma.shape) == (n_layers, d), f"norm_gamma must be [{n_layers}][{d}]")
    for b_, nm in ((k_bias, "k_bias"), (v_bias, "v_bias")):
        if b_ is not None:
            _need(tuple(b_.shape) == (n_layers, n_out), f"{nm} must be [{n_layers}][{n_out}]")
    if pos is not None:
        _need(pos.dim() == 1 and pos.shape[0] >= n_rows, "pos must hold one position per row of h")
        _need(rope_cos is not None and rope_sin is not None and
              tuple(rope_cos.shape) == tuple(rope_sin.shape) and rope_cos.shape[1] == head_dim // 2,
              f"rope_cos and rope_sin must both be [n_pos][{head_dim // 2}]")
    dk = w4(*wk)
    dv = w4(*wv)
    lay = RiverLayer(_ptr(norm_gamma), norm_eps, _ptr(k_bias), _ptr(v_bias), _ptr(pos),
                     _ptr(rope_cos), _ptr(rope_sin),
                     rope_cos.shape[0] if rope_cos is not None else 0)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().river_kv_fill_layer(m_max, _ptr(m_dev), d, _dt(h), _ptr(h), _ld(h), n_rows,
                                      _ptr(row_idx), _ptr(slot), n_layers, _ptr(maps),
                                      ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(lay),
                                      n_kv_heads, head_dim, _ptr(k_cache), _ptr(v_cache),
                                      k_cache.shape[1], _ptr(workspace), ws_n, _stream(stream)))


def _decode_args(checkpoints, wk, wv, n_kv_heads, head_dim, slot, k_cache, v_cache, exit_layer, gamma,
                 eps, rule):
    """The C arguments of a decode step up to exit_layer (checked), and the
    descriptors they point to (kept alive by the caller)."""
    h0 = checkpoints[0]["h_cur"]
    n, d = h0.shape
    ld = _ld(h0)
    b = 0
    n_layers = k_cache.shape[0]
    n_out = n_kv_heads * head_dim
    _check_w4(wk, n_layers, n_out, d, "wk")
    _check_w4(wv, n_layers, n_out, d, "wv")
    for cch, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(cch.dim() == 4 and tuple(cch.shape[2:]) == (n_kv_heads, head_dim) and cch.is_contiguous(),
              f"{nm} must be contiguous [n_layers][n_slots][{n_kv_heads}][{head_dim}]")
    _need(tuple(k_cache.shape) == tuple(v_cache.shape), "k_cache and v_cache must have the same shape")
    _need(slot.dim() == 1 and slot.shape[0] >= n, f"slot must hold one entry per token ({n})")
    _need(exit_layer.numel() >= n, f"exit_layer must hold one entry per token ({n})")
    arr = (RiverCheckpoint * len(checkpoints))()
    for i, c in enumerate(checkpoints):
        if _ld(c["h_prev"]) != ld or _ld(c["h_cur"]) != ld:
            raise ValueError("every state must have the same leading dimension")
        _need(c["h_prev"].shape[0] >= n and c["h_cur"].shape[0] >= n,
              f"checkpoint {i}: states must hold {n} rows")
        mp = c.get("maps")
        if mp is not None:
            e = int(c["layer"])
            _need(tuple(mp.shape) == (n_layers - e, d, d) and mp.is_contiguous(),
                  f"checkpoint {i}: maps must be contiguous [{n_layers - e}][{d}][{d}]")
        fo = c.get("folded")
        if fo is not None:
            e = int(c["layer"])
            _need(tuple(fo.shape) == (n_layers - e, 2 * n_out, d) and fo.is_contiguous() and
                  _dt(fo) == RIVER_BF16,
                  f"checkpoint {i}: folded must be contiguous bf16 [{n_layers - e}][{2 * n_out}][{d}]")
        wd = c.get("w_down")
        if wd is not None:
            b = wd.shape[0]
        arr[i] = RiverCheckpoint(int(c["layer"]), _ptr(c["h_prev"]), _ptr(c["h_cur"]),
                                 float(c["tau"]), float(c["theta"]), _ptr(wd), _ptr(c.get("w_up")),
                                 _ptr(c.get("maps")), _ptr(c.get("folded")))
    dk = w4(*wk)
    dv = w4(*wv)
    args = (n, d, _dt(h0), ld, len(checkpoints), arr, n_layers, _ptr(gamma), eps, b, rule,
            ctypes.byref(dk), ctypes.byref(dv), n_kv_heads, head_dim, _ptr(slot), _ptr(k_cache),
            _ptr(v_cache), k_cache.shape[1], _ptr(exit_layer))
    return args, (arr, dk, dv)


def river_decode_step(checkpoints, wk, wv, n_kv_heads, head_dim, slot, k_cache, v_cache,
                      exit_layer, *, gamma=None, eps=1e-6, rule=RULE_TOKEN, workspace=None,
                      stream=None):
    """checkpoints: list of dicts with layer, h_prev, h_cur, tau, theta and
    optionally w_down, w_up, maps; wk, wv: (q, scale, zero, group) of every
    block; caches [n_layers][n_slots][Hkv][Dh]."""
    args, keep = _decode_args(checkpoints, wk, wv, n_kv_heads, head_dim, slot, k_cache, v_cache,
                              exit_layer, gamma, eps, rule)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().river_decode_step(*args, _ptr(workspace), ws_n, _stream(stream)))
    del keep


def river_decode_step_static(checkpoints, wk, wv, n_kv_heads, head_dim, slot, k_cache, v_cache,
                             exit_layer, *, gamma=None, eps=1e-6, rule=RULE_TOKEN, stream=None):
    """river_decode_step on the library's static device scratch (no
    workspace, nothing allocated)."""
    args, keep = _decode_args(checkpoints, wk, wv, n_kv_heads, head_dim, slot, k_cache, v_cache,
                              exit_layer, gamma, eps, rule)
    _check(load().river_decode_step_static(*args, _stream(stream)))
    del keep


def river_router_fit(h, labels, w_down, w_up, *, epochs=100, batch=256, order=None, gamma=None,
                     eps=1e-6, lr=1e-3, beta1=0.9, beta2=0.999, adam_eps=1e-8, loss_out=None,
                     workspace=None, stream=None):
    """w_down (fp32 [b][d]) and w_up (fp32 [b]) are trained in place."""
    n, d = h.shape
    b = w_down.shape[0]
    _need(tuple(w_down.shape) == (b, d) and w_down.is_contiguous(), f"w_down must be contiguous [b][{d}]")
    _need(w_up.numel() == b, f"w_up must hold b = {b} entries")
    _need(labels.numel() >= n, f"labels must hold {n} entries")
    if order is not None:
        _need(order.numel() >= epochs * n, f"order must hold epochs x n = {epochs * n} entries")
    if loss_out is not None:
        _need(loss_out.numel() >= epochs, f"loss_out must hold {epochs} entries")
    if workspace is None:
        raise ValueError("river_router_fit needs a workspace (river_workspace_size(OP_ROUTER_FIT, ...))")
    ws_n = workspace.numel() * workspace.element_size()
    _check(load().river_router_fit(n, d, _dt(h), _ptr(h), _ld(h), _ptr(labels), _ptr(gamma), eps, b,
                                   _ptr(w_down), _ptr(w_up), epochs, batch, _ptr(order), lr, beta1,
                                   beta2, adam_eps, _ptr(loss_out), _ptr(workspace), ws_n,
                                   _stream(stream)))


def river_ridge_fit(X, Y, lam, W, *, workspace=None, stream=None):
    n, d_in = X.shape
    n_targets, n_y, d_out = Y.shape
    _need(n_y == n, f"Y must be [n_targets][{n}][d_out] (one row per calibration token), got {tuple(Y.shape)}")
    _need(tuple(W.shape) == (n_targets, d_out, d_in),
          f"W must be [{n_targets}][{d_out}][{d_in}], got {tuple(W.shape)}")
    _need(X.is_contiguous() and Y.is_contiguous() and W.is_contiguous(), "X, Y and W must be contiguous")
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().river_ridge_fit(n, d_in, d_out, n_targets, _ptr(X), _dt(X), _ptr(Y), _dt(Y),
                                  lam, _ptr(W), _dt(W), _ptr(workspace), ws_n, _stream(stream)))
