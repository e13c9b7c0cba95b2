"""Pins for the oracle's layer pieces (CPU only).

Each check ties the oracle to something other than itself: the partition
identities the pages state (MLM-notes, "Model Parallel Transformers"; PAR-survey,
"How": column split = output dim, row split = input dim; heads independent),
closed forms, brute force on tiny inputs, central finite differences, and
independent library routines (torch's float64 GeLU, LayerNorm, scaled
dot-product attention, multi-head attention and autograd).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as tF

import oracle as O

RNG = np.random.default_rng(1234)


def rnd(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def t64(a):
    return torch.tensor(a, dtype=torch.float64)


# ----------------------------------------------------------------- GeLU

def test_gelu_closed_forms():
    z = rnd(200) * 3
    assert O.gelu(np.array([0.0]))[0] == 0.0
    assert np.allclose(O.gelu(-z), O.gelu(z) - z, rtol=0, atol=1e-14)
    # GeLU(1) = Phi(1) through libm's erf (a separate path from scipy's).
    assert abs(O.gelu(np.array([1.0]))[0] - 0.5 * (1 + math.erf(1 / math.sqrt(2)))) < 1e-15
    assert np.array_equal(O.gelu(z, "none"), z)


@pytest.mark.parametrize("mode,approx", [("erf", "none"), ("tanh", "tanh")])
def test_gelu_matches_torch(mode, approx):
    z = rnd(1000) * 4
    ref = tF.gelu(t64(z), approximate=approx).numpy()
    assert np.allclose(O.gelu(z, mode), ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("mode", ["erf", "tanh", "none"])
def test_gelu_grad_finite_difference(mode):
    z = rnd(300) * 3
    h = 1e-6
    fd = (O.gelu(z + h, mode) - O.gelu(z - h, mode)) / (2 * h)
    assert np.allclose(O.gelu_grad(z, mode), fd, rtol=1e-7, atol=1e-8)


# ----------------------------------------------------------- LayerNorm

def test_layernorm_matches_torch_and_closed_form():
    x = rnd(9, 33) * 2 + 0.5
    g, b = rnd(33), rnd(33)
    y, mean, rstd = O.layernorm(x, g, b, 1e-5)
    ref = tF.layer_norm(t64(x), (33,), t64(g), t64(b), 1e-5).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    # gamma = 1, beta = 0: each row has mean 0 and variance var/(var + eps).
    y1, _, _ = O.layernorm(x, np.ones(33), np.zeros(33), 1e-5)
    var = x.var(axis=1)
    assert np.allclose(y1.mean(axis=1), 0, atol=1e-13)
    assert np.allclose(y1.var(axis=1), var / (var + 1e-5), rtol=1e-12)


def test_layernorm_bwd_against_autograd_and_fd():
    x, g, b, dy = rnd(5, 17), rnd(17), rnd(17), rnd(5, 17)
    _, mean, rstd = O.layernorm(x, g, b)
    dx, dg, db = O.layernorm_bwd(dy, x, g, mean, rstd)
    xt, gt, bt = (t64(v).requires_grad_() for v in (x, g, b))
    tF.layer_norm(xt, (17,), gt, bt, 1e-5).backward(t64(dy))
    assert np.allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dg, gt.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(db, bt.grad.numpy(), rtol=1e-10, atol=1e-12)
    v = rnd(5, 17)
    h = 1e-6
    f = lambda xx: (O.layernorm(xx, g, b)[0] * dy).sum()
    fd = (f(x + h * v) - f(x - h * v)) / (2 * h)
    assert abs(fd - (dx * v).sum()) < 1e-6 * max(1.0, abs(fd))


# ------------------------------------------------ column / row linears

def brute_column(x, a, bias, act):
    t, k = x.shape
    f = a.shape[0]
    y = np.zeros((t, f))
    for i in range(t):
        for j in range(f):
            acc = bias[j]
            for kk in range(k):
                acc += x[i, kk] * a[j, kk]
            y[i, j] = acc
    return O.gelu(y, act)


def test_column_linear_brute_force_and_one_hot():
    x, a, bias = rnd(3, 5), rnd(4, 5), rnd(4)
    y, z = O.column_linear(x, a, bias, "erf")
    assert np.allclose(y, brute_column(x, a, bias, "erf"), rtol=1e-13, atol=1e-14)
    # One-hot rows of X return the matching columns of A (plus the bias).
    eye = np.eye(5)
    y0, _ = O.column_linear(eye, a, bias, "none")
    assert np.allclose(y0, a.T + bias, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [1, 2, 4])
def test_column_split_concatenates(n):
    x, a, bias = rnd(6, 16), rnd(32, 16), rnd(32)
    full, _ = O.column_linear(x, a, bias)
    fi = 32 // n
    parts = [O.column_linear(x, a[i * fi:(i + 1) * fi], bias[i * fi:(i + 1) * fi])[0] for i in range(n)]
    assert np.allclose(np.concatenate(parts, axis=1), full, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("n", [1, 2, 4])
def test_row_split_partials_sum(n):
    y, b = rnd(6, 32), rnd(16, 32)
    full = y @ b.T
    fi = 32 // n
    parts = [O.row_linear_partial(y[:, i * fi:(i + 1) * fi], b[:, i * fi:(i + 1) * fi]) for i in range(n)]
    assert np.allclose(sum(parts), full, rtol=1e-13, atol=1e-13)
    if n == 1:
        assert np.allclose(parts[0], full, rtol=1e-15, atol=0)


def _dir_fd(f, x, v, h=1e-6):
    return (f(x + h * v) - f(x - h * v)) / (2 * h)


@pytest.mark.parametrize("act", ["erf", "tanh", "none"])
def test_column_linear_bwd_fd(act):
    x, a, bias, dy = rnd(4, 6), rnd(5, 6), rnd(5), rnd(4, 5)
    _, z = O.column_linear(x, a, bias, act)
    dx, da, dbias = O.column_linear_bwd(x, a, z, dy, act)
    for arg, grad in ((0, dx), (1, da), (2, dbias)):
        args = [x, a, bias]
        v = rnd(*args[arg].shape)

        def f(val, arg=arg):
            cur = list(args)
            cur[arg] = val
            return (O.column_linear(*cur, act)[0] * dy).sum()
        assert abs(_dir_fd(f, args[arg], v) - (grad * v).sum()) < 1e-6


def test_row_linear_bwd_fd():
    y, b, dout = rnd(4, 6), rnd(5, 6), rnd(4, 5)
    dy, db = O.row_linear_partial_bwd(y, b, dout)
    v = rnd(4, 6)
    assert abs(_dir_fd(lambda q: (O.row_linear_partial(q, b) * dout).sum(), y, v) - (dy * v).sum()) < 1e-6
    v = rnd(5, 6)
    assert abs(_dir_fd(lambda q: (O.row_linear_partial(y, q) * dout).sum(), b, v) - (db * v).sum()) < 1e-6


# ------------------------------------------------------- shard reduce

def test_shard_reduce_integer_partials_exact():
    parts = [RNG.integers(-1000, 1000, size=(8, 12)).astype(np.float64) for _ in range(8)]
    bias = RNG.integers(-10, 10, size=12).astype(np.float64)
    res = RNG.integers(-10, 10, size=(8, 12)).astype(np.float64)
    out, keep = O.shard_reduce(parts, bias, res, 0.0)
    assert keep.all()
    want = np.zeros((8, 12))
    for i in range(8):
        for j in range(12):
            want[i, j] = res[i, j] + bias[j] + sum(pp[i, j] for pp in parts)
    assert np.array_equal(out, want)


def test_shard_reduce_dropout_and_bwd():
    parts = [rnd(6, 10) for _ in range(3)]
    bias, res = rnd(10), rnd(6, 10)
    out, keep = O.shard_reduce(parts, bias, res, 0.2, 9, 4)
    mask = O.dropout_keep_mask(60, 0.2, 9, 4).reshape(6, 10)
    assert np.array_equal(keep, mask)
    scale = 1 / (1 - float(np.float32(0.2)))
    assert np.allclose(out, res + np.where(mask, (sum(parts) + bias) * scale, 0), rtol=1e-15, atol=1e-15)
    dout = rnd(6, 10)
    d_pre, d_bias = O.shard_reduce_bwd(dout, 0.2, 9, 4)
    v = rnd(6, 10)
    f = lambda q: (O.shard_reduce([q] + parts[1:], bias, res, 0.2, 9, 4)[0] * dout).sum()
    assert abs(_dir_fd(f, parts[0], v) - (d_pre * v).sum()) < 1e-6
    assert np.allclose(d_bias, d_pre.sum(0))


# --------------------------------------------------------- attention

def _sdpa(q, k, v, causal):
    return tF.scaled_dot_product_attention(t64(q), t64(k), t64(v), is_causal=causal).numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_attention_matches_torch_sdpa(causal):
    q, k, v = rnd(2, 3, 9, 8), rnd(2, 3, 9, 8), rnd(2, 3, 9, 8)
    o, lse = O.attention_core(q, k, v, causal)
    assert np.allclose(o, _sdpa(q, k, v, causal), rtol=1e-12, atol=1e-13)
    s = np.einsum("bhld,bhmd->bhlm", q, k) / math.sqrt(8)
    if causal:
        s = np.where(np.tril(np.ones((9, 9), bool)), s, -np.inf)
    assert np.allclose(lse, torch.logsumexp(t64(s), dim=-1).numpy(), rtol=1e-13, atol=1e-13)


def test_attention_closed_forms():
    v = rnd(1, 2, 7, 4)
    # Q = 0: every visible key has equal weight -> causal prefix mean of V.
    o, lse = O.attention_core(np.zeros((1, 2, 7, 4)), rnd(1, 2, 7, 4), v, True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, 8)[None, None, :, None]
    assert np.allclose(o, prefix, rtol=1e-14, atol=1e-14)
    assert np.allclose(lse, np.log(np.arange(1, 8))[None, None, :], atol=1e-14)
    # L = 1: the only key is the token itself -> O = V.
    v1 = rnd(2, 3, 1, 4)
    o1, _ = O.attention_core(rnd(2, 3, 1, 4), rnd(2, 3, 1, 4), v1, True)
    assert np.allclose(o1, v1, rtol=0, atol=1e-15)


def test_attention_brute_force_loops():
    q, k, v = rnd(1, 1, 4, 3), rnd(1, 1, 4, 3), rnd(1, 1, 4, 3)
    o, _ = O.attention_core(q, k, v, True)
    for l in range(4):
        w = [math.exp(sum(q[0, 0, l, e] * k[0, 0, m, e] for e in range(3)) / math.sqrt(3))
             for m in range(l + 1)]
        tot = sum(w)
        for e in range(3):
            assert abs(o[0, 0, l, e] - sum(w[m] * v[0, 0, m, e] for m in range(l + 1)) / tot) < 1e-13


@pytest.mark.parametrize("causal", [True, False])
def test_attention_bwd_matches_autograd(causal):
    q, k, v, do = rnd(2, 2, 6, 4), rnd(2, 2, 6, 4), rnd(2, 2, 6, 4), rnd(2, 2, 6, 4)
    dq, dk, dv = O.attention_core_bwd(q, k, v, do, causal)
    qt, kt, vt = (t64(a).requires_grad_() for a in (q, k, v))
    tF.scaled_dot_product_attention(qt, kt, vt, is_causal=causal).backward(t64(do))
    for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        assert np.allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_head_attention_matches_torch_mha():
    # Full-head case (K = heads * d): torch's packed in-projection uses the
    # same [Q; K; V] row blocks with contiguous per-head slices.
    bsz, seq, heads, d = 2, 5, 3, 4
    kdim = heads * d
    x, w, bq = rnd(bsz * seq, kdim), rnd(3 * kdim, kdim, scale=0.3), rnd(3 * kdim)
    wo, bo = rnd(kdim, kdim, scale=0.3), rnd(kdim)
    ctx, _, _ = O.head_attention(x, w, bq, bsz, seq, heads, d, True)
    ours = O.row_linear_partial(ctx, wo) + bo
    xs = t64(x.reshape(bsz, seq, kdim)).transpose(0, 1)
    mask = torch.triu(torch.ones(seq, seq, dtype=torch.bool), 1)
    ref, _ = tF.multi_head_attention_forward(
        xs, xs, xs, kdim, heads, t64(w), t64(bq), None, None, False, 0.0, t64(wo), t64(bo),
        training=False, need_weights=False, attn_mask=mask)
    ref = ref.transpose(0, 1).reshape(bsz * seq, kdim).numpy()
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n", [1, 3])
def test_head_split_equals_full_mha(n):
    bsz, seq, heads, d, kdim = 2, 6, 6, 4, 10
    x, w, bq, wo = rnd(bsz * seq, kdim), rnd(3 * heads * d, kdim, scale=0.3), rnd(3 * heads * d), rnd(kdim, heads * d)
    ctx, _, _ = O.head_attention(x, w, bq, bsz, seq, heads, d)
    full = O.row_linear_partial(ctx, wo)
    hi, hd = heads // n, heads * d
    parts, ctxs = [], []
    for i in range(n):
        rows = np.concatenate([np.arange(b * hd + i * hi * d, b * hd + (i + 1) * hi * d) for b in range(3)])
        c_i, _, _ = O.head_attention(x, w[rows], bq[rows], bsz, seq, hi, d)
        ctxs.append(c_i)
        parts.append(O.row_linear_partial(c_i, wo[:, i * hi * d:(i + 1) * hi * d]))
    assert np.allclose(np.concatenate(ctxs, axis=1), ctx, rtol=1e-13, atol=1e-14)
    assert np.allclose(sum(parts), full, rtol=1e-12, atol=1e-13)


def test_head_attention_bwd_fd():
    bsz, seq, heads, d, kdim = 1, 4, 2, 3, 5
    x, w, bq, dctx = rnd(bsz * seq, kdim), rnd(3 * heads * d, kdim, scale=0.5), rnd(3 * heads * d), rnd(bsz * seq, heads * d)
    _, _, qkv = O.head_attention(x, w, bq, bsz, seq, heads, d)
    dx, dw, db = O.head_attention_bwd(x, w, qkv, dctx, bsz, seq, heads, d)
    for idx, grad in ((0, dx), (1, dw), (2, db)):
        args = [x, w, bq]
        v = rnd(*args[idx].shape)

        def f(val, idx=idx):
            cur = list(args)
            cur[idx] = val
            return (O.head_attention(*cur, bsz, seq, heads, d)[0] * dctx).sum()
        assert abs(_dir_fd(f, args[idx], v) - (grad * v).sum()) < 1e-6


# ------------------------------------------------------------ full layer

def tiny_layer(kdim=12, heads=3, d=4, f=24):
    prm = {"ln1_g": 1 + rnd(kdim, scale=0.1), "ln1_b": rnd(kdim, scale=0.1),
           "w_qkv": rnd(3 * heads * d, kdim, scale=0.3), "b_qkv": rnd(3 * heads * d, scale=0.1),
           "w_o": rnd(kdim, heads * d, scale=0.3), "b_o": rnd(kdim, scale=0.1),
           "ln2_g": 1 + rnd(kdim, scale=0.1), "ln2_b": rnd(kdim, scale=0.1),
           "w_a": rnd(f, kdim, scale=0.3), "b_a": rnd(f, scale=0.1),
           "w_b": rnd(kdim, f, scale=0.3), "b_b": rnd(kdim, scale=0.1)}
    return prm


def test_layer_forward_matches_torch_modules():
    bsz, seq, heads, d, kdim = 2, 5, 3, 4, 12
    prm = tiny_layer(kdim, heads, d)
    x = rnd(bsz * seq, kdim)
    c = O.layer_forward(prm, x, bsz, seq, heads, d, p=0.0)
    T = {k: t64(v) for k, v in prm.items()}
    xt = t64(x)
    h = tF.layer_norm(xt, (kdim,), T["ln1_g"], T["ln1_b"], 1e-5)
    hs = h.reshape(bsz, seq, kdim).transpose(0, 1)
    mask = torch.triu(torch.ones(seq, seq, dtype=torch.bool), 1)
    att, _ = tF.multi_head_attention_forward(hs, hs, hs, kdim, heads, T["w_qkv"], T["b_qkv"], None, None,
                                             False, 0.0, T["w_o"], T["b_o"], training=False,
                                             need_weights=False, attn_mask=mask)
    h1 = xt + att.transpose(0, 1).reshape(bsz * seq, kdim)
    h2 = tF.layer_norm(h1, (kdim,), T["ln2_g"], T["ln2_b"], 1e-5)
    out = h1 + tF.linear(tF.gelu(tF.linear(h2, T["w_a"], T["b_a"])), T["w_b"], T["b_b"])
    assert np.allclose(c["out"], out.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("p", [0.0, 0.3])
def test_layer_backward_fd(p):
    bsz, seq, heads, d, kdim = 1, 4, 2, 3, 6
    prm = tiny_layer(kdim, heads, d, 10)
    x, dout = rnd(bsz * seq, kdim), rnd(bsz * seq, kdim)
    kw = dict(p=p, seed=77, offsets=(3, 8))
    c = O.layer_forward(prm, x, bsz, seq, heads, d, **kw)
    g = O.layer_backward(prm, x, c, dout, bsz, seq, heads, d, **kw)

    def loss(pr, xx):
        return (O.layer_forward(pr, xx, bsz, seq, heads, d, **kw)["out"] * dout).sum()
    v = rnd(*x.shape)
    assert abs(_dir_fd(lambda q: loss(prm, q), x, v) - (g["x"] * v).sum()) < 1e-6
    for name in prm:
        v = rnd(*prm[name].shape)

        def f(val, name=name):
            pr = dict(prm)
            pr[name] = val
            return loss(pr, x)
        fd = _dir_fd(f, prm[name], v)
        assert abs(fd - (g[name] * v).sum()) < 1e-6 * max(1.0, abs(fd)), name


@pytest.mark.parametrize("n", [2, 3])
def test_layer_rank_shards_compose(n):
    # The per-rank pieces, with the shard reduce standing in for the all-reduce,
    # give the unpartitioned layer (forward and the input gradient).
    bsz, seq, heads, d, kdim, f = 2, 4, 6, 2, 8, 12
    prm = tiny_layer(kdim, heads, d, f)
    x, dout = rnd(bsz * seq, kdim), rnd(bsz * seq, kdim)
    kw = dict(p=0.25, seed=5, offsets=(1, 2))
    c = O.layer_forward(prm, x, bsz, seq, heads, d, **kw)
    g = O.layer_backward(prm, x, c, dout, bsz, seq, heads, d, **kw)
    hi, hd, fi = heads // n, heads * d, f // n
    shards = []
    for i in range(n):
        rows = np.concatenate([np.arange(b * hd + i * hi * d, b * hd + (i + 1) * hi * d) for b in range(3)])
        shards.append(dict(w_qkv=prm["w_qkv"][rows], b_qkv=prm["b_qkv"][rows],
                           w_o=prm["w_o"][:, i * hi * d:(i + 1) * hi * d],
                           w_a=prm["w_a"][i * fi:(i + 1) * fi], b_a=prm["b_a"][i * fi:(i + 1) * fi],
                           w_b=prm["w_b"][:, i * fi:(i + 1) * fi]))
    h, mu1, rs1 = O.layernorm(x, prm["ln1_g"], prm["ln1_b"])
    att = [O.head_attention(h, s["w_qkv"], s["b_qkv"], bsz, seq, hi, d) for s in shards]
    h1, _ = O.shard_reduce([O.row_linear_partial(a[0], s["w_o"]) for a, s in zip(att, shards)],
                           prm["b_o"], x, 0.25, 5, 1)
    h2, mu2, rs2 = O.layernorm(h1, prm["ln2_g"], prm["ln2_b"])
    mlp = [O.column_linear(h2, s["w_a"], s["b_a"]) for s in shards]
    out, _ = O.shard_reduce([O.row_linear_partial(m[0], s["w_b"]) for m, s in zip(mlp, shards)],
                            prm["b_b"], h1, 0.25, 5, 2)
    assert np.allclose(out, c["out"], rtol=1e-12, atol=1e-12)
    # Backward: the conjugate reduces of the column layers' input-gradient partials.
    d_mlp, _ = O.shard_reduce_bwd(dout, 0.25, 5, 2)
    dh2 = []
    for m, s in zip(mlp, shards):
        dy_i, _ = O.row_linear_partial_bwd(m[0], s["w_b"], d_mlp)
        dh2.append(O.column_linear_bwd(h2, s["w_a"], m[1], dy_i)[0])
    dh1 = dout + O.layernorm_bwd(sum(dh2), h1, prm["ln2_g"], mu2, rs2)[0]
    d_att, _ = O.shard_reduce_bwd(dh1, 0.25, 5, 1)
    dh = []
    for a, s in zip(att, shards):
        dctx, _ = O.row_linear_partial_bwd(a[0], s["w_o"], d_att)
        dh.append(O.head_attention_bwd(h, s["w_qkv"], a[2], dctx, bsz, seq, hi, d)[0])
    dx = dh1 + O.layernorm_bwd(sum(dh), x, prm["ln1_g"], mu1, rs1)[0]
    assert np.allclose(dx, g["x"], rtol=1e-11, atol=1e-12)
