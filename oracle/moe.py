"""Oracle of one expert-parallel shard of a MoE layer (fp64).

Test infrastructure only (see the package docstring).  MOE-core, technical
summary: section 1 (routing, permutation and dynamic shapes of fine-grained
experts), section 2.4 (grouped GEMM: all experts' products batched into one
kernel; sync-free kernels read the dynamic shapes on the device) and section
2.2 (memory-efficient permutation).  The router itself is an input here: the
top-k expert ids and their weights are given.

Readings: an expert is a SwiGLU FFN, ``silu(x W_g^T) * (x W_u^T)`` followed by
``W_d``, with the gate rows first and the up rows second in ``W_gu``; the
routing weight is applied when the expert outputs are summed back per token
(the "unpermute with routing weights" form), or, in the memory-efficient
variant of section 2.2, to the expert's activation before its down projection
(so the unpermute is a plain sum and the backward needs no saved expert
output); the two agree in exact arithmetic because the down projection is
linear.  The permutation lists the local picks expert-major, then by token,
then by slot.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def moe_permutation(topk_ids, e_start, e_local):
    """Enumerate this shard's picks.

    Experts ``e_start .. e_start + e_local - 1`` are local.  Returns
    ``(counts [e_local], offsets [e_local + 1], picks [R])`` where ``picks``
    holds the flat pick index ``t * topk + k`` of every local pick, ordered by
    local expert, then token, then slot; ``offsets`` is the exclusive prefix
    sum of ``counts``.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    tokens, topk = ids.shape
    counts = np.zeros(e_local, dtype=np.int64)
    picks = []
    for e in range(e_local):
        for t in range(tokens):
            for k in range(topk):
                if ids[t, k] == e_start + e:
                    picks.append(t * topk + k)
                    counts[e] += 1
    offsets = np.zeros(e_local + 1, dtype=np.int64)
    for e in range(e_local):
        offsets[e + 1] = offsets[e] + counts[e]
    return counts, offsets, np.asarray(picks, dtype=np.int64)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def expert_swiglu_ffn(x, w_gu, w_d):
    """One expert on rows ``x [R, Hd]``: ``(silu(x W_g^T) * (x W_u^T)) W_d^T``
    with ``W_g = w_gu[:Fe]``, ``W_u = w_gu[Fe:]``, ``w_d [Hd, Fe]``."""
    x, w_gu, w_d = _f64(x), _f64(w_gu), _f64(w_d)
    fe = w_d.shape[1]
    gate = x @ w_gu[:fe].T
    up = x @ w_gu[fe:].T
    return (_silu(gate) * up) @ w_d.T


def moe_forward_rows(x, topk_ids, topk_w, w_gu, w_d, e_start, tokens):
    """The shard's output for the listed ``tokens`` only:
    ``out[t] = sum_k [ids[t,k] local] w[t,k] * FFN_{ids[t,k]}(x_t)``, summed
    over k ascending; tokens with no local pick give zeros."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = _f64(topk_w)
    e_local = np.shape(w_gu)[0]
    x = _f64(x)
    out = np.zeros((len(tokens), x.shape[1]))
    for i, t in enumerate(tokens):
        for k in range(ids.shape[1]):
            e = ids[t, k] - e_start
            if 0 <= e < e_local:
                out[i] += w[t, k] * expert_swiglu_ffn(x[t:t + 1], w_gu[e], w_d[e])[0]
    return out


def moe_forward(x, topk_ids, topk_w, w_gu, w_d, e_start):
    """Whole-shard forward: permute by expert, run each local expert on its
    rows, sum back per token with the routing weights.  Returns
    ``(out [T, Hd], counts, offsets, picks, y_perm [R, Hd])``."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    tokens, topk = ids.shape
    w = _f64(topk_w)
    x = _f64(x)
    e_local = np.shape(w_gu)[0]
    counts, offsets, picks = moe_permutation(ids, e_start, e_local)
    y_perm = np.zeros((picks.size, x.shape[1]))
    for e in range(e_local):
        sel = picks[offsets[e]:offsets[e + 1]]
        if sel.size:
            y_perm[offsets[e]:offsets[e + 1]] = expert_swiglu_ffn(x[sel // topk], w_gu[e], w_d[e])
    out = np.zeros_like(x)
    row_of = {int(pk): r for r, pk in enumerate(picks)}
    for t in range(tokens):
        for k in range(topk):
            r = row_of.get(t * topk + k)
            if r is not None:
                out[t] += w[t, k] * y_perm[r]
    return out, counts, offsets, picks, y_perm


def moe_forward_weighted_act(x, topk_ids, topk_w, w_gu, w_d, e_start):
    """Memory-efficient permutation form of :func:`moe_forward` (MOE-core,
    technical summary 2.2: the routing weight is applied before the expert's
    activation leaves it, here to the SwiGLU activation ahead of the down
    projection).  Row ``r`` of the permuted activation is
    ``w[pick_r] * silu(g_r) * u_r``; ``y_perm = act W_d^T``; the unpermute
    sums ``y_perm`` rows per token without weights.  Returns
    ``(out [T, Hd], counts, offsets, picks, y_perm [R, Hd])``."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    tokens, topk = ids.shape
    w = _f64(topk_w).reshape(-1)
    x = _f64(x)
    e_local = np.shape(w_gu)[0]
    counts, offsets, picks = moe_permutation(ids, e_start, e_local)
    y_perm = np.zeros((picks.size, x.shape[1]))
    for e in range(e_local):
        sel = picks[offsets[e]:offsets[e + 1]]
        if sel.size:
            wgu, wd = _f64(w_gu[e]), _f64(w_d[e])
            fe = wd.shape[1]
            xe = x[sel // topk]
            act = _silu(xe @ wgu[:fe].T) * (xe @ wgu[fe:].T)
            act = act * w[sel][:, None]
            y_perm[offsets[e]:offsets[e + 1]] = act @ wd.T
    out = np.zeros_like(x)
    for r, pk in enumerate(picks):
        out[int(pk) // topk] += y_perm[r]
    return out, counts, offsets, picks, y_perm


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def moe_backward(x, topk_ids, topk_w, w_gu, w_d, e_start, dout):
    """Backward of :func:`moe_forward` (the weighted-unpermute form) for the
    upstream gradient ``dout [T, Hd]`` of the shard's output.

    MOE-core, technical summary 2.4: the backward runs the same grouped
    structure, per local expert over its permuted rows.  For a local pick
    ``(t, k)`` of expert ``e`` with ``g = x_t W_g^T``, ``u = x_t W_u^T``,
    ``a = silu(g) * u`` and ``y = a W_d^T``:

    * ``dy = w[t,k] * dout_t`` and ``d w[t,k] = dout_t . y``;
    * ``da = dy W_d`` and ``dW_d += dy^T a``;
    * ``dg = da * u * silu'(g)`` with ``silu'(g) = s (1 + g (1 - s))``,
      ``s = sigmoid(g)``, and ``du = da * silu(g)``;
    * ``dW_g += dg^T x_t``, ``dW_u += du^T x_t``, ``dx_t += dg W_g + du W_u``.

    Picks on other shards get ``d w = 0`` and add nothing to ``dx``.  Returns
    a dict with ``x [T, Hd]``, ``w_gu [E, 2Fe, Hd]``, ``w_d [E, Hd, Fe]`` and
    ``topk_w [T, topk]``.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    tokens, topk = ids.shape
    w = _f64(topk_w).reshape(-1)
    x, dout = _f64(x), _f64(dout)
    w_gu, w_d = _f64(w_gu), _f64(w_d)
    e_local, _, fe = w_d.shape
    counts, offsets, picks = moe_permutation(ids, e_start, e_local)
    dx = np.zeros_like(x)
    dw_gu = np.zeros_like(w_gu)
    dw_d = np.zeros_like(w_d)
    dw = np.zeros(tokens * topk)
    for e in range(e_local):
        sel = picks[offsets[e]:offsets[e + 1]]
        if sel.size == 0:
            continue
        tok = sel // topk
        xe = x[tok]
        wg, wu, wd = w_gu[e, :fe], w_gu[e, fe:], w_d[e]
        g = xe @ wg.T
        u = xe @ wu.T
        s = _sigmoid(g)
        a = g * s * u
        y = a @ wd.T
        dy = w[sel][:, None] * dout[tok]
        dw[sel] = np.sum(dout[tok] * y, axis=1)
        da = dy @ wd
        dw_d[e] = dy.T @ a
        dg = da * u * s * (1.0 + g * (1.0 - s))
        du = da * g * s
        dw_gu[e, :fe] = dg.T @ xe
        dw_gu[e, fe:] = du.T @ xe
        dxe = dg @ wg + du @ wu
        for i, t in enumerate(tok):
            dx[t] += dxe[i]
    return {"x": dx, "w_gu": dw_gu, "w_d": dw_d, "topk_w": dw.reshape(tokens, topk)}


def moe_backward_weighted_act(x, topk_ids, topk_w, w_gu, w_d, e_start, dout):
    """Backward of :func:`moe_forward_weighted_act`, the memory-efficient
    permutation form (MOE-core, technical summary 2.2: with the routing
    weight applied before the expert's output is formed, the backward needs
    no saved expert output).  For a local pick ``(t, k)`` of expert ``e``
    with ``g``, ``u``, ``s = sigmoid(g)``, the unweighted activation
    ``a = silu(g) * u`` and the weighted one ``a_w = w[t,k] * a``:

    * ``dy = dout_t`` (the unpermute is an unweighted sum);
    * ``d a_w = dy W_d`` and ``dW_d += dy^T a_w``;
    * ``d w[t,k] = d a_w . a`` (the weight's gradient from the activation
      side), ``d a = w[t,k] * d a_w``;
    * ``dg``, ``du``, ``dW_gu`` and ``dx`` as in :func:`moe_backward`.

    Equal to :func:`moe_backward` in exact arithmetic (both differentiate the
    same function).  Returns the same dict.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    tokens, topk = ids.shape
    w = _f64(topk_w).reshape(-1)
    x, dout = _f64(x), _f64(dout)
    w_gu, w_d = _f64(w_gu), _f64(w_d)
    e_local, _, fe = w_d.shape
    counts, offsets, picks = moe_permutation(ids, e_start, e_local)
    dx = np.zeros_like(x)
    dw_gu = np.zeros_like(w_gu)
    dw_d = np.zeros_like(w_d)
    dw = np.zeros(tokens * topk)
    for e in range(e_local):
        sel = picks[offsets[e]:offsets[e + 1]]
        if sel.size == 0:
            continue
        tok = sel // topk
        xe = x[tok]
        wg, wu, wd = w_gu[e, :fe], w_gu[e, fe:], w_d[e]
        g = xe @ wg.T
        u = xe @ wu.T
        s = _sigmoid(g)
        a = g * s * u
        a_w = w[sel][:, None] * a
        dy = dout[tok]
        da_w = dy @ wd
        dw_d[e] = dy.T @ a_w
        dw[sel] = np.sum(da_w * a, axis=1)
        da = w[sel][:, None] * da_w
        dg = da * u * s * (1.0 + g * (1.0 - s))
        du = da * g * s
        dw_gu[e, :fe] = dg.T @ xe
        dw_gu[e, fe:] = du.T @ xe
        dxe = dg @ wg + du @ wu
        for i, t in enumerate(tok):
            dx[t] += dxe[i]
    return {"x": dx, "w_gu": dw_gu, "w_d": dw_d, "topk_w": dw.reshape(tokens, topk)}
