"""Oracle of one transformer layer and of its tensor-parallel pieces (fp64).

Test infrastructure only (see the package docstring).  Conventions: tokens are
flattened ``t = b * L + l`` into rows of ``[T, K]`` matrices; every weight is
stored ``[out, in]``; the fused QKV weight holds the Q rows of all its heads,
then the K rows, then the V rows, ``d`` consecutive rows per head.
"""

import math

import numpy as np
from scipy.special import erf

from .philox import dropout


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Element-wise pieces
# --------------------------------------------------------------------------

def gelu(z, mode="erf"):
    """GeLU.  The pages name GeLU in the MLP split (MLM-notes, "Model Parallel
    Transformers", MLP paragraph) without defining it; reading: the exact
    definition ``z * Phi(z) = z * (1 + erf(z / sqrt 2)) / 2``.  ``mode="tanh"``
    is the common tanh approximation, kept as a library option."""
    z = _f64(z)
    if mode == "erf":
        return z * 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
    if mode == "tanh":
        c = math.sqrt(2.0 / math.pi)
        return 0.5 * z * (1.0 + np.tanh(c * (z + 0.044715 * z ** 3)))
    if mode == "none":
        return z.copy()
    raise ValueError(mode)


def gelu_grad(z, mode="erf"):
    """Derivative of :func:`gelu`: ``Phi(z) + z * phi(z)`` for the exact form."""
    z = _f64(z)
    if mode == "erf":
        cdf = 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
        pdf = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
        return cdf + z * pdf
    if mode == "tanh":
        c = math.sqrt(2.0 / math.pi)
        u = c * (z + 0.044715 * z ** 3)
        t = np.tanh(u)
        return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3 * 0.044715 * z * z)
    if mode == "none":
        return np.ones_like(z)
    raise ValueError(mode)


def layernorm(x, gamma, beta, eps=1e-5):
    """LayerNorm over the last axis (MLM-review, "approach" section: LayerNorm
    placement matters for deep BERT-like models; the pages give no formula).
    Reading: biased variance, ``eps = 1e-5``.  Returns ``(y, mean, rstd)``."""
    x = _f64(x)
    mean = x.mean(axis=-1)
    var = ((x - mean[..., None]) ** 2).mean(axis=-1)
    rstd = 1.0 / np.sqrt(var + eps)
    y = (x - mean[..., None]) * rstd[..., None] * _f64(gamma) + _f64(beta)
    return y, mean, rstd


def layernorm_bwd(dy, x, gamma, mean, rstd):
    """Chain rule of :func:`layernorm`.  Returns ``(dx, dgamma, dbeta)``."""
    dy, x, gamma = _f64(dy), _f64(x), _f64(gamma)
    xhat = (x - mean[..., None]) * rstd[..., None]
    g = dy * gamma
    k = x.shape[-1]
    dx = rstd[..., None] * (g - g.sum(-1, keepdims=True) / k
                            - xhat * (g * xhat).sum(-1, keepdims=True) / k)
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def bias_grad(dy):
    """Gradient of a bias added to every row: the column sums of ``dy``."""
    return _f64(dy).sum(axis=0)


# --------------------------------------------------------------------------
# Column- and row-parallel linears
# --------------------------------------------------------------------------

def column_linear(x, a_w, a_b=None, act="erf"):
    """Column-parallel linear: the weight is split along its output dimension
    (PAR-survey, "How", tensor parallelism; MLM-notes, "Model Parallel
    Transformers", MLP paragraph), so a rank holding rows ``A_i`` of ``A``
    produces the column slice ``act(X A_i^T + a_i)`` of the full output.
    Returns ``(Y, Z)`` with ``Z`` the pre-activation."""
    z = _f64(x) @ _f64(a_w).T
    if a_b is not None:
        z = z + _f64(a_b)
    return gelu(z, act), z


def column_linear_bwd(x, a_w, z, dy, act="erf"):
    """Backward of :func:`column_linear`.  ``dX`` is a full-shape *partial*
    (each rank's share of the input gradient; summing the shares is the
    backward all-reduce, MLM-notes "Model Parallel Transformers", communication
    paragraph).  Returns ``(dX_partial, dA, da)``."""
    dz = _f64(dy) * gelu_grad(z, act)
    return dz @ _f64(a_w), dz.T @ _f64(x), dz.sum(axis=0)


def row_linear_partial(y, b_w):
    """Row-parallel linear: the weight is split along its input dimension
    (PAR-survey, "How"; MLM-notes, "Model Parallel Transformers"), so a rank
    holding columns ``B_i`` of ``B`` produces a full-shape partial
    ``Y_i B_i^T``; the partials sum to ``Y B^T``.  No bias here: a bias is
    added once, after the sum."""
    return _f64(y) @ _f64(b_w).T


def row_linear_partial_bwd(y, b_w, dout):
    """Backward of :func:`row_linear_partial`: ``dY_i = dOut B_i`` and
    ``dB_i = dOut^T Y_i``; ``dOut`` is replicated on every rank."""
    dout = _f64(dout)
    return dout @ _f64(b_w), dout.T @ _f64(y)


def shard_reduce(partials, bias=None, residual=None, p=0.0, seed=0, offset=0):
    """``out = residual + Drop(sum_j partials[j] + bias)``.

    The sum over shards is the all-reduce after each partitioned block
    (MLM-notes, "Model Parallel Transformers": one all-reduce completes the
    layer; MLM-review, "approach": results merged by all-reduce).  The dropout
    is the synchronised one (MLM-review, "key terms"), indexed by the flat
    position in the full ``[rows, cols]`` tensor.  Returns ``(out, keep)``."""
    acc = np.zeros(np.shape(partials[0]), dtype=np.float64)
    for part in partials:
        acc = acc + _f64(part)
    if bias is not None:
        acc = acc + _f64(bias)
    y, keep = dropout(acc, p, seed, offset)
    if residual is not None:
        y = y + _f64(residual)
    return y, keep


def shard_reduce_bwd(dout, p=0.0, seed=0, offset=0):
    """Backward of :func:`shard_reduce`.  Returns ``(d_pre, d_bias)``: the
    gradient of every partial (and of the sum) is ``Drop(dout)`` with the same
    mask; the residual's gradient is ``dout`` itself."""
    d_pre, _ = dropout(dout, p, seed, offset)
    return d_pre, d_pre.sum(axis=0)


# --------------------------------------------------------------------------
# Head-partitioned attention
# --------------------------------------------------------------------------

def split_qkv_heads(qkv, batch, seq, heads, d):
    """View the fused ``[T, 3*heads*d]`` projection as Q, K, V ``[B, h, L, d]``."""
    q = _f64(qkv).reshape(batch, seq, 3, heads, d)
    return (q[:, :, 0].transpose(0, 2, 1, 3), q[:, :, 1].transpose(0, 2, 1, 3),
            q[:, :, 2].transpose(0, 2, 1, 3))


def attention_core(q, k, v, causal=True):
    """Scaled dot-product attention per (batch, head), heads independent
    (MLM-notes, "Model Parallel Transformers", attention paragraph).  Reading:
    scale ``1/sqrt(d)``; the causal mask keeps key ``m <= l`` for query ``l``.
    ``q, k, v`` are ``[B, h, L, d]``; returns ``(O, lse)`` with ``lse`` the
    natural log of each softmax normaliser, ``[B, h, L]``."""
    bsz, nh, seq, d = q.shape
    scale = 1.0 / math.sqrt(d)
    out = np.empty_like(q)
    lse = np.empty((bsz, nh, seq))
    mask = np.tril(np.ones((seq, seq), dtype=bool)) if causal else None
    for b in range(bsz):
        for h in range(nh):
            s = (q[b, h] @ k[b, h].T) * scale
            if causal:
                s = np.where(mask, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            den = e.sum(axis=1, keepdims=True)
            out[b, h] = (e / den) @ v[b, h]
            lse[b, h] = (m + np.log(den))[:, 0]
    return out, lse


def attention_core_bwd(q, k, v, do, causal=True):
    """Chain rule of :func:`attention_core` (P recomputed from its
    definition).  Returns ``(dq, dk, dv)``."""
    bsz, nh, seq, d = q.shape
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    mask = np.tril(np.ones((seq, seq), dtype=bool)) if causal else None
    for b in range(bsz):
        for h in range(nh):
            s = (q[b, h] @ k[b, h].T) * scale
            if causal:
                s = np.where(mask, s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            pr = e / e.sum(axis=1, keepdims=True)
            dv[b, h] = pr.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            ds = pr * (dp - (dp * pr).sum(axis=1, keepdims=True))
            dq[b, h] = ds @ k[b, h] * scale
            dk[b, h] = ds.T @ q[b, h] * scale
    return dq, dk, dv


def _heads_to_rows(o):
    bsz, nh, seq, d = o.shape
    return o.transpose(0, 2, 1, 3).reshape(bsz * seq, nh * d)


def _rows_to_heads(x, batch, seq, heads, d):
    return _f64(x).reshape(batch, seq, heads, d).transpose(0, 2, 1, 3)


def head_attention(x, w_qkv, b_qkv, batch, seq, heads, d, causal=True):
    """One rank's attention: the fused QKV product for its ``heads`` heads,
    then attention per head (MLM-review, "approach": the Q, K, V products are
    split across GPUs; MLM-notes: heads are assigned to GPUs).  Returns
    ``(ctx [T, heads*d], lse [B, heads, L], qkv [T, 3*heads*d])``."""
    qkv = _f64(x) @ _f64(w_qkv).T
    if b_qkv is not None:
        qkv = qkv + _f64(b_qkv)
    q, k, v = split_qkv_heads(qkv, batch, seq, heads, d)
    o, lse = attention_core(q, k, v, causal)
    return _heads_to_rows(o), lse, qkv


def head_attention_bwd(x, w_qkv, qkv, dctx, batch, seq, heads, d, causal=True):
    """Backward of :func:`head_attention`.  Returns
    ``(dX_partial, dW_qkv, db_qkv)``; ``dX_partial`` is this rank's share of
    the input gradient."""
    q, k, v = split_qkv_heads(qkv, batch, seq, heads, d)
    do = _rows_to_heads(dctx, batch, seq, heads, d)
    dq, dk, dv = attention_core_bwd(q, k, v, do, causal)
    dqkv = np.concatenate([_heads_to_rows(dq), _heads_to_rows(dk), _heads_to_rows(dv)], axis=1)
    return dqkv @ _f64(w_qkv), dqkv.T @ _f64(x), dqkv.sum(axis=0)


# --------------------------------------------------------------------------
# Whole layer (unpartitioned)
# --------------------------------------------------------------------------

def layer_forward(prm, x, batch, seq, heads, d, p=0.0, seed=0, offsets=(0, 1),
                  causal=True, act="erf", eps=1e-5):
    """Pre-LN transformer layer, the unpartitioned computation that the shards
    compose to.

    ``H1 = X + Drop(Attn(LN1(X)) W_o^T + b_o)``;
    ``Out = H1 + Drop(GeLU(LN2(H1) A^T + a) B^T + b)``.

    Attention and MLP per MLM-notes, "Model Parallel Transformers"; dropout
    synchronised per MLM-review, "key terms".  Readings: pre-LN placement
    (GPT-2-style block), biases on every linear, dropout on the two residual
    branches only.  ``prm`` holds ``ln1_g, ln1_b, w_qkv, b_qkv, w_o, b_o,
    ln2_g, ln2_b, w_a, b_a, w_b, b_b``.  Returns a dict of intermediates.
    """
    c = {}
    c["h"], c["mu1"], c["rs1"] = layernorm(x, prm["ln1_g"], prm["ln1_b"], eps)
    c["ctx"], c["lse"], c["qkv"] = head_attention(c["h"], prm["w_qkv"], prm["b_qkv"],
                                                  batch, seq, heads, d, causal)
    attn = row_linear_partial(c["ctx"], prm["w_o"])
    c["h1"], c["keep1"] = shard_reduce([attn], prm["b_o"], x, p, seed, offsets[0])
    c["h2"], c["mu2"], c["rs2"] = layernorm(c["h1"], prm["ln2_g"], prm["ln2_b"], eps)
    c["y"], c["z"] = column_linear(c["h2"], prm["w_a"], prm["b_a"], act)
    mlp = row_linear_partial(c["y"], prm["w_b"])
    c["out"], c["keep2"] = shard_reduce([mlp], prm["b_b"], c["h1"], p, seed, offsets[1])
    return c


def layer_backward(prm, x, c, dout, batch, seq, heads, d, p=0.0, seed=0,
                   offsets=(0, 1), causal=True, act="erf"):
    """Exact chain rule of :func:`layer_forward` for upstream ``dout``.
    Returns a dict with ``dx`` and the gradient of every parameter."""
    g = {}
    dout = _f64(dout)
    d_mlp, g["b_b"] = shard_reduce_bwd(dout, p, seed, offsets[1])
    dy, g["w_b"] = row_linear_partial_bwd(c["y"], prm["w_b"], d_mlp)
    dh2, g["w_a"], g["b_a"] = column_linear_bwd(c["h2"], prm["w_a"], c["z"], dy, act)
    dh1_ln, g["ln2_g"], g["ln2_b"] = layernorm_bwd(dh2, c["h1"], prm["ln2_g"], c["mu2"], c["rs2"])
    dh1 = dout + dh1_ln
    d_attn, g["b_o"] = shard_reduce_bwd(dh1, p, seed, offsets[0])
    dctx, g["w_o"] = row_linear_partial_bwd(c["ctx"], prm["w_o"], d_attn)
    dh, g["w_qkv"], g["b_qkv"] = head_attention_bwd(c["h"], prm["w_qkv"], c["qkv"], dctx,
                                                    batch, seq, heads, d, causal)
    dx_ln, g["ln1_g"], g["ln1_b"] = layernorm_bwd(dh, x, prm["ln1_g"], c["mu1"], c["rs1"])
    g["x"] = dh1 + dx_ln
    return g
