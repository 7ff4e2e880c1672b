"""Float64 NumPy oracle of the per-token exit-and-KV-fill step.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
CPU-baseline leg of the benchmark; never by the product path.

Each function is the plain definition of one operation, written from the
pages' description (cited per function) in float64 from the exact values of
the fp32 or bf16 inputs. There is no blocking, fusion or reordering beyond
what the definition states. Where the pages leave a step open the reading
taken is stated in the docstring.

Conventions shared with the library's C interface (these are layout
contracts, not arithmetic):

* hidden states are row-major ``[n][d]``; one row per token;
* a linear map ``M`` of shape ``[d_out][d_in]`` acts as
  ``x_hat[j] = sum_k M[j][k] * x[k]`` (the output-major layout of a weight
  matrix);
* int4 weights ``q`` are ``[n_out][k/2]`` bytes, element ``k`` in byte
  ``k // 2``, low nibble when ``k`` is even; scale and zero are
  ``[n_out][k/group]``; the dequantized value is ``(q - zero) * scale``;
* caches are ``[layer][slot][n_kv_heads][head_dim]``.
"""

import numpy as np

RULE_TOKEN = 0
RULE_BATCH_MIN = 1


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _sigmoid(z):
    # logistic function 1 / (1 + e^-z); e^-z may overflow to inf for very
    # negative z, which gives exactly 0 as the limit requires.
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def route(h_prev, h_cur, gamma, eps, w_down, w_up, tau, theta, rule=RULE_TOKEN):
    """Exit decision for every token of a batch.

    Sources:
      * River-LLM, "前置知识" (state transition similarity): the cosine
        between a block's input h^(l-1) and output h^(l) of the same token.
      * River-LLM, "方法步骤详情" step 3: a token may exit when the
        similarity exceeds tau; the batch form takes the minimum over the
        batch. Step 3's closing sentence and the weakness list propose
        independent per-token decisions (rule TOKEN).
      * TIDE, "关键公式" formula 3 (Router MLP): phi(h) = sigmoid(W_up .
        SiLU(W_down . RMSNorm(h))) with W_down in R^{b x d}, W_up in
        R^{1 x b}, no biases (the parameter count d*b + b in "系统架构" is
        exactly the two matrices).
      * TIDE, formula 4: exit when phi exceeds theta (strict), for every
        token of the batch (rule BATCH_MIN).

    Readings taken: RMSNorm is h * gamma / sqrt(mean(h^2) + eps) over the d
    features; the router reads h^(l) (the state after the block); the two
    tests are combined with AND; a comparison with NaN is false, so a NaN
    token continues; a zero norm gives cos = 0; cos is clamped to [-1, 1].
    ``w_down=None`` switches the router off: prob is 1 and only the cosine
    test applies.

    Returns (cos[n], prob[n], mask[n] uint8, all_exit int); all_exit is the
    AND of the per-token decisions (0 for an empty batch).
    """
    a = _f64(h_prev)
    b = _f64(h_cur)
    n, d = b.shape
    # cosine: a.b / (|a| |b|)
    dot = np.sum(a * b, axis=1)
    na = np.sum(a * a, axis=1)
    nb = np.sum(b * b, axis=1)
    cos = np.zeros(n)
    ok = (na > 0) & (nb > 0)
    with np.errstate(invalid="ignore"):
        cos[ok] = dot[ok] / np.sqrt(na[ok] * nb[ok])
    bad = ~((na > 0) | (na == 0)) | ~((nb > 0) | (nb == 0))  # NaN norms
    cos[bad] = np.nan
    cos = np.clip(cos, -1.0, 1.0)

    if w_down is None:
        prob = np.ones(n)
        with np.errstate(invalid="ignore"):
            e = cos > tau
    else:
        g = np.ones(d) if gamma is None else _f64(gamma)
        # RMSNorm over the feature dimension
        r = 1.0 / np.sqrt(nb / d + eps)
        x = b * g[None, :] * r[:, None]
        u = x @ _f64(w_down).T            # [n][b]   W_down . RMSNorm(h)
        act = u * _sigmoid(u)             # SiLU(u) = u * sigma(u)
        z = act @ _f64(w_up).reshape(-1)  # W_up . SiLU(...)
        prob = _sigmoid(z)
        with np.errstate(invalid="ignore"):
            e = (cos > tau) & (prob > theta)

    all_exit = int(n > 0 and bool(np.all(e)))
    if rule == RULE_BATCH_MIN:
        mask = np.full(n, all_exit, dtype=np.uint8)
    elif rule == RULE_TOKEN:
        mask = e.astype(np.uint8)
    else:
        raise ValueError("unknown rule")
    return cos, prob, mask, all_exit


def compact(mask, h, row_ids=None, out=None):
    """Stable split of a batch into continuing and exiting tokens.

    Source: TIDE, "模块4: 融合 CUDA 内核" -- Batch Compact separates the
    continuing tokens from the exiting ones; Exit Scatter copies the exited
    tokens' hidden states back to their original positions in an output
    buffer.

    Definition: cont = ascending i with mask[i] == 0, exit = ascending i with
    mask[i] != 0; h_cont[j] = h[cont[j]], row_ids_cont[j] = row_ids[cont[j]];
    out[row_ids[exit[j]]] = h[exit[j]]. ``row_ids=None`` means the identity.
    ``out`` (optional) is copied and the scatter applied to the copy.
    """
    mask = np.asarray(mask)
    n = mask.shape[0]
    cont, ext = [], []
    for i in range(n):
        if mask[i] != 0:
            ext.append(i)
        else:
            cont.append(i)
    cont = np.array(cont, dtype=np.int64)
    ext = np.array(ext, dtype=np.int64)
    rid = np.arange(n, dtype=np.int64) if row_ids is None else np.asarray(row_ids, dtype=np.int64)
    res = {
        "cont_idx": cont,
        "exit_idx": ext,
        "counts": np.array([len(cont), len(ext)], dtype=np.int64),
        "row_ids_cont": rid[cont] if n else rid[:0],
    }
    if h is not None:
        h = np.asarray(h)
        res["h_cont"] = h[cont] if n else h[:0]
        if out is not None:
            o = np.array(out, copy=True)
            for i in ext:
                o[rid[i]] = h[i]
            res["out"] = o
    return res


def exit_projection(h, row_idx, m, gamma, eps, out, row_ids=None):
    """Final RMSNorm of the exited rows, scattered to their original places.

    Source: TIDE, "模块4: 融合 CUDA 内核" -- Exit Projection fuses an RMSNorm
    with the scatter of exited tokens; "模块3: Post-Hoc Generation" -- an
    exited token's logits come from the LM head applied to the RMSNorm of
    its hidden state, so this is the state handed to the LM head.

    Definition, for t = 0..m-1 with r = row_idx[t] (or t when row_idx is
    None) and dst = row_ids[r] (or r when row_ids is None):

        out[dst][j] = gamma[j] * h[r][j] / sqrt(mean_k(h[r][k]^2) + eps)

    Readings taken: the mean runs over the d features; gamma=None means all
    ones; rows r outside [0, n) and destinations outside [0, len(out)) are
    skipped (the library's convention for out-of-range indices); every other
    row of ``out`` is left as given. A zero row with eps = 0 gives 0/0 = NaN,
    as IEEE arithmetic does. ``out`` is copied and the copy returned (float64).
    """
    h = _f64(h)
    n, d = h.shape
    g = np.ones(d) if gamma is None else _f64(gamma)
    o = _f64(out).copy()
    for t in range(int(m)):
        r = t if row_idx is None else int(row_idx[t])
        if not (0 <= r < n):
            continue
        dst = r if row_ids is None else int(row_ids[r])
        if not (0 <= dst < o.shape[0]):
            continue
        x = h[r]
        ms = np.mean(x * x)
        with np.errstate(divide="ignore", invalid="ignore"):
            o[dst] = g * x / np.sqrt(ms + eps)
    return o


def dequant_w4(q, scale, zero, group):
    """Dequantize group-quantized int4 weights: w = (q - zero) * scale.

    Source: River-LLM, "前置知识" (PTQ): W4A16 keeps 4-bit weights with
    16-bit activations. The group form, asymmetric with a scale and a zero
    point per ``group`` input channels of each output row, is the reading
    taken (the page's HQQ quantizer is not reproduced; only its storage form
    is).

    q: uint8 [..., n_out, k/2], element k in byte k//2, low nibble if k even.
    scale, zero: [..., n_out, k/group]. Returns float64 [..., n_out, k].
    """
    q = np.asarray(q, dtype=np.uint8)
    lo = (q & 0x0F).astype(np.float64)
    hi = (q >> 4).astype(np.float64)
    k2 = q.shape[-1]
    vals = np.empty(q.shape[:-1] + (2 * k2,), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    s = np.repeat(_f64(scale), group, axis=-1)
    z = np.repeat(_f64(zero), group, axis=-1)
    return (vals - z) * s


def kv_fill_rows(h, row_idx, m, maps, wk, wv):
    """K and V rows that a fill writes, per skipped layer.

    Sources:
      * RidgeFill, method paragraph under "思路源头": after the split layer,
        every later layer's input is predicted from the split-layer state
        with a fitted map, and that layer's own projection writes the cache.
      * River-LLM, "方法步骤详情" step 1 and "核心方法": the exit path of a
        token produces the K/V of every skipped layer with a W4A16 copy of
        the layer's weights.
      * River-LLM, "研究动机" (State Propagation) and RidgeFill's identity
        fill baseline: the map may be the identity.

    Reading taken: "the layer's projection" is the linear K and V
    projection only (no input norm, no RoPE, no bias).

    h: [rows][d]; row_idx: indices of the m rows to fill (None: 0..m-1);
    maps: None (identity) or [n_layers][d][d] output-major; wk, wv: dicts
    with q [n_layers][n_out][d/2], scale, zero [n_layers][n_out][d/group],
    group. Returns (K, V), each float64 [n_layers][m][n_out].
    """
    h = _f64(h)
    rows = np.arange(m) if row_idx is None else np.asarray(row_idx, dtype=np.int64)[:m]
    x = h[rows]                                   # [m][d]
    n_layers = np.asarray(wk["q"]).shape[0]
    n_out = np.asarray(wk["q"]).shape[1]
    K = np.empty((n_layers, m, n_out))
    V = np.empty((n_layers, m, n_out))
    for l in range(n_layers):
        xh = x if maps is None else x @ _f64(maps[l]).T   # x_hat = M x
        Wk = dequant_w4(wk["q"][l], wk["scale"][l], wk["zero"][l], wk["group"])
        Wv = dequant_w4(wv["q"][l], wv["scale"][l], wv["zero"][l], wv["group"])
        K[l] = xh @ Wk.T
        V[l] = xh @ Wv.T
    return K, V


def rope_half(x, cos, sin):
    """Rotary position embedding of head vectors, half-split pairing.

    Not defined on the pages: this is the standard rotary embedding
    (RoFormer) in the layout of Llama-family models, the models River-LLM
    evaluates; it is part of "the layer's own projection" whose output the
    cache holds (RidgeFill, "思路源头").

    x: [..., hd]; cos, sin: [..., hd/2], broadcast against x. Element i is
    paired with element i + hd/2 and the pair is turned by the angle whose
    cosine and sine are cos[i] and sin[i]:
        y[i] = x[i] cos[i] - x[i + hd/2] sin[i]
        y[i + hd/2] = x[i] sin[i] + x[i + hd/2] cos[i]
    """
    x = _f64(x)
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    c, s = _f64(cos), _f64(sin)
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def kv_fill_layer_rows(h, row_idx, m, maps, wk, wv, gamma=None, eps=0.0, bk=None, bv=None,
                       pos=None, cos=None, sin=None, n_kv_heads=None, head_dim=None):
    """K and V rows of a fill through the skipped layers' full K/V path.

    Sources: RidgeFill, "思路源头": the predicted input of a skipped layer
    goes through that layer's own projection, which writes the cache as it
    normally would. River-LLM, "方法步骤详情" step 1: the K/V are those of
    the skipped layer, at the backbone's addresses.

    Reading taken: the layer's usual K/V path is its input RMSNorm (weight
    gamma[l], over the d features, as TIDE's RMSNorm), the K and V linear
    maps with optional biases bk[l], bv[l] (GPT-2-style), then rotary
    position embedding of K only, per head, at the row's position
    (``rope_half``; pos is indexed by the row of h, tables cos/sin are
    [n_pos][head_dim/2]). Any of the three may be absent (None).

    Returns (K, V), each float64 [n_layers][m][n_out].
    """
    h = _f64(h)
    rows = np.arange(m) if row_idx is None else np.asarray(row_idx, dtype=np.int64)[:m]
    x = h[rows]
    n_layers = np.asarray(wk["q"]).shape[0]
    n_out = np.asarray(wk["q"]).shape[1]
    K = np.empty((n_layers, m, n_out))
    V = np.empty((n_layers, m, n_out))
    for l in range(n_layers):
        xh = x if maps is None else x @ _f64(maps[l]).T        # predicted layer input
        if gamma is not None:                                  # the layer's input RMSNorm
            ms = np.mean(xh * xh, axis=1)
            xh = _f64(gamma[l])[None, :] * xh / np.sqrt(ms + eps)[:, None]
        Wk = dequant_w4(wk["q"][l], wk["scale"][l], wk["zero"][l], wk["group"])
        Wv = dequant_w4(wv["q"][l], wv["scale"][l], wv["zero"][l], wv["group"])
        K[l] = xh @ Wk.T
        V[l] = xh @ Wv.T
        if bk is not None:
            K[l] += _f64(bk[l])[None, :]
        if bv is not None:
            V[l] += _f64(bv[l])[None, :]
        if pos is not None:                                    # RoPE on K, per head
            p = np.asarray(pos, dtype=np.int64)[rows]
            k = K[l].reshape(m, n_kv_heads, head_dim)
            c = _f64(cos)[p][:, None, :]
            sn = _f64(sin)[p][:, None, :]
            K[l] = rope_half(k, c, sn).reshape(m, n_out)
    return K, V


def kv_fill(h, row_idx, m, slot, maps, wk, wv, n_kv_heads, head_dim, k_cache, v_cache):
    """Write K/V of every skipped layer into each exited token's own slot.

    Source: River-LLM, "方法步骤详情" step 1 and "技术新颖性": the exit path
    writes K/V at exactly the addresses the backbone would use (position
    index, head split, dimension layout), so the cache stays complete
    ("Intrinsic KV Integrity", "研究动机"). Values as in ``kv_fill_rows``.

    slot is indexed by the row of h: token row r goes to slot[r] of every
    layer. Returns new float64 caches [n_layers][n_slots][Hkv][Dh]; the
    inputs are not modified; untouched slots keep their values.
    """
    K, V = kv_fill_rows(h, row_idx, m, maps, wk, wv)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    rows = np.arange(m) if row_idx is None else np.asarray(row_idx, dtype=np.int64)[:m]
    slot = np.asarray(slot, dtype=np.int64)
    for l in range(K.shape[0]):
        for t in range(m):
            s = slot[rows[t]]
            kc[l, s] = K[l, t].reshape(n_kv_heads, head_dim)
            vc[l, s] = V[l, t].reshape(n_kv_heads, head_dim)
    return kc, vc


def decode_step(checkpoints, n_layers, rule, slot, wk, wv, n_kv_heads, head_dim, k_cache,
                v_cache, gamma=None, eps=1e-6):
    """One generation step of the token-level exit loop over checkpoints.

    Source: River-LLM, "方法步骤详情" step 3: during generation each token's
    state climbs the blocks; after block l the state-transition similarity
    decides whether the token switches to the exit path, which then writes
    the K/V of every remaining block at that token's slot (step 1). TIDE
    "模块4" / formula 4 give the per-token decision with a router; River
    takes the minimum over the batch (``RULE_BATCH_MIN``).

    checkpoints: list, in increasing layer order, of dicts with
      layer (e, 1 <= e < L), h_prev (h^(e-1), [n][d]), h_cur (h^(e)),
      tau, theta, w_down / w_up (None: router off), maps (None: identity,
      else [L - e][d][d]).
    wk, wv: int4 descriptors of blocks 1..L (``n_layers`` = L layers);
    caches: [L][n_slots][Hkv][Dh], cache layer j - 1 holding block j.

    Readings taken: a token takes part in a checkpoint only while it has
    not exited; it exits at the first checkpoint whose decision passes
    (under the batch rule: every still-running token passes); its exit state
    is h_cur of that checkpoint and blocks e+1..L are filled from it as in
    ``kv_fill``. Tokens that never exit get exit layer L.
    Returns (exit_layer int64 [n], k_cache, v_cache) (caches copied).
    """
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    n = np.asarray(checkpoints[0]["h_cur"]).shape[0]
    alive = np.ones(n, dtype=bool)
    exit_layer = np.full(n, n_layers, dtype=np.int64)
    for ck in checkpoints:
        e = int(ck["layer"])
        _, _, m, _ = route(ck["h_prev"], ck["h_cur"], gamma, eps, ck.get("w_down"),
                           ck.get("w_up"), ck["tau"], ck["theta"], RULE_TOKEN)
        dec = (m != 0) & alive
        if rule == RULE_BATCH_MIN:
            every = alive.any() and bool(np.all(dec[alive]))
            dec = alive & every
        rows = np.flatnonzero(dec)
        exit_layer[rows] = e
        alive &= ~dec
        if len(rows):
            sub = lambda w: {"q": np.asarray(w["q"])[e:], "scale": np.asarray(w["scale"])[e:],
                             "zero": np.asarray(w["zero"])[e:], "group": w["group"]}
            kc[e:], vc[e:] = kv_fill(ck["h_cur"], rows, len(rows), slot, ck.get("maps"), sub(wk),
                                     sub(wv), n_kv_heads, head_dim, kc[e:], vc[e:])
    return exit_layer, kc, vc


def router_labels(h_k, h_final, tau_c=0.98):
    """Calibration labels of one checkpoint.

    Source: TIDE, "模块1: 离线校准": a token counts as converged at checkpoint
    k when the cosine between its state there and its final-layer state
    exceeds the convergence threshold (0.98 by default, "关键公式" formula 1).
    Returns uint8 [n] (1 = converged); the cosine follows ``route``'s rules
    (zero norm gives 0, NaN compares false).
    """
    cos, _, _, _ = route(h_final, h_k, None, 0.0, None, None, tau_c, -np.inf)
    return (cos > tau_c).astype(np.uint8)


def router_fit(h, labels, w_down, w_up, epochs, batch, order=None, gamma=None, eps=1e-6,
               lr=1e-3, beta1=0.9, beta2=0.999, adam_eps=1e-8):
    """Train one checkpoint's router with binary cross-entropy and Adam.

    Source: TIDE, "模块1: 离线校准" and the experiment settings: the two-layer
    router of formula 3 (RMSNorm, W_down, SiLU, w_up, sigmoid) is trained on
    the calibration states with the BCE loss and Adam (lr = 1e-3) for 100
    epochs.

    Readings taken: mini-batches of ``batch`` tokens in the order ``order[e]``
    (a permutation per epoch, drawn by the caller; None: 0..n-1), the last
    batch of an epoch possibly shorter; the loss of a batch is the mean of
    -[y log p + (1 - y) log(1 - p)] over its tokens; Adam as published by
    Kingma and Ba (first and second moments, bias correction with the global
    step count, no weight decay), defaults beta1 = 0.9, beta2 = 0.999,
    eps = 1e-8; the RMSNorm weight is fixed (not trained: the router's
    parameters are the two matrices). Gradients are the chain rule through
    z = w_up . SiLU(u), u = W_down . x, x = gamma * h / rms(h):
        dL/dz_i = (sigmoid(z_i) - y_i) / B
        dL/dw_up = sum_i dL/dz_i SiLU(u_i)
        dL/du_i = dL/dz_i * w_up * SiLU'(u_i),  SiLU'(u) = s(u) (1 + u (1 - s(u)))
        dL/dW_down = sum_i dL/du_i x_i^T

    Returns (w_down [b][d], w_up [b], mean loss per epoch [epochs]), float64.
    """
    h = _f64(h)
    n, d = h.shape
    y = np.asarray(labels, dtype=np.float64)
    g = np.ones(d) if gamma is None else _f64(gamma)
    W = _f64(w_down).copy()
    w = _f64(w_up).copy()
    mW, vW = np.zeros_like(W), np.zeros_like(W)
    mw, vw = np.zeros_like(w), np.zeros_like(w)
    r = 1.0 / np.sqrt(np.mean(h * h, axis=1) + eps)
    X = h * g[None, :] * r[:, None]                  # RMSNorm of every token
    t = 0
    losses = np.zeros(epochs)
    for e in range(epochs):
        idx = np.arange(n) if order is None else np.asarray(order[e], dtype=np.int64)
        total = 0.0
        for s0 in range(0, n, batch):
            rows = idx[s0:s0 + batch]
            B = len(rows)
            x, yy = X[rows], y[rows]
            u = x @ W.T                                # [B][b]
            su = _sigmoid(u)
            a = u * su                                 # SiLU
            z = a @ w                                  # [B]
            p = _sigmoid(z)
            # BCE from the logit: softplus(z) - y z
            total += float(np.sum(np.logaddexp(0.0, z) - yy * z))
            gz = (p - yy) / B
            gw = a.T @ gz
            gu = gz[:, None] * w[None, :] * (su * (1.0 + u * (1.0 - su)))
            gW = gu.T @ x
            t += 1
            for P, G, M, V in ((W, gW, mW, vW), (w, gw, mw, vw)):
                M *= beta1
                M += (1.0 - beta1) * G
                V *= beta2
                V += (1.0 - beta2) * G * G
                mh = M / (1.0 - beta1 ** t)
                vh = V / (1.0 - beta2 ** t)
                P -= lr * mh / (np.sqrt(vh) + adam_eps)
        losses[e] = total / n
    return W, w, losses


def ridge_fit(X, Y, lam):
    """Closed-form ridge maps, one per target.

    Source: RidgeFill, closed-form ridge regression box: W = (X^T X +
    lambda I)^-1 X^T Y, fitted once from a single calibration pass, X the
    split-layer states and Y a later layer's inputs.

    Readings taken: no intercept; lambda is not scaled by n. The result is
    returned output-major, W_out[t] = W_t^T of shape [d_out][d_in], so that
    x_hat = W_out[t] x is the row form x_hat^T = x^T W_t.

    X: [n][d_in]; Y: [T][n][d_out]. Returns float64 [T][d_out][d_in].
    """
    X = _f64(X)
    Y = _f64(Y)
    d_in = X.shape[1]
    G = X.T @ X + lam * np.eye(d_in)
    out = np.empty((Y.shape[0], Y.shape[2], d_in))
    for t in range(Y.shape[0]):
        W = np.linalg.solve(G, X.T @ Y[t])      # [d_in][d_out]
        out[t] = W.T
    return out


def exit_schedule_ops(exit_layers, n_layers):
    """Layer operations of a per-token exit schedule.

    Source: TIDE, "Figure 2" (per-token early exit in a 32-layer model): a
    token that exits after block e executes e blocks and skips the rest.

    Blocks are numbered 1..L; exit at e runs blocks 1..e; the skipped blocks
    e+1..L each need a K/V fill (River-LLM, "研究动机": the skipped layers
    otherwise leave no K/V). Returns executed, baseline (every token runs L
    blocks), filled (token-layers filled) and the fractional reduction.
    """
    e = [int(x) for x in exit_layers]
    for x in e:
        if not (1 <= x <= n_layers):
            raise ValueError("exit layer out of range")
    executed = sum(e)
    baseline = len(e) * n_layers
    filled = sum(n_layers - x for x in e)
    return {
        "executed": executed,
        "baseline": baseline,
        "filled": filled,
        "reduction": (baseline - executed) / baseline if baseline else 0.0,
    }
