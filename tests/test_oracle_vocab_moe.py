"""Pins for the oracle's vocab-parallel and MoE pieces (CPU only).

Vocab: the split lookup sums to the full lookup exactly (MLM-notes, "Model
Parallel Transformers", embedding paragraph); per-shard exponentials and row
sums combine to the full softmax normaliser (output paragraph); closed forms
(zero logits give ln V; a shift of all logits changes nothing); torch's
float64 cross-entropy and autograd as independent library routines.

MoE (MOE-core, technical summary 2.2 and 2.4): the permutation is pinned
against numpy's stable argsort; the expert FFN against a hand-computed scalar
case and a brute-force loop; the permuted forward against the per-token
definition; the memory-efficient form (weight on the activation) against the
weighted-unpermute form, which linearity of the down projection makes equal;
the backward against central finite differences of the per-token forward and
against torch's float64 autograd of a per-token forward written in torch ops.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as tF

import oracle as O

RNG = np.random.default_rng(4321)


def rnd(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


@pytest.mark.parametrize("n", [1, 2, 8])
def test_embedding_split_sums_exactly(n):
    v, k, t = 64, 5, 40
    emb = rnd(v, k)
    ids = RNG.integers(0, v, size=t)
    vi = v // n
    parts = [O.vocab_parallel_embedding(ids, emb[i * vi:(i + 1) * vi], i * vi) for i in range(n)]
    total = np.zeros((t, k))
    for part in parts:
        total = total + part
    assert np.array_equal(total, O.embedding(ids, emb))
    assert np.array_equal(O.embedding(ids, emb), emb[ids])


@pytest.mark.parametrize("n", [1, 4])
def test_embedding_backward_is_the_lookup_adjoint(n):
    # <lookup(E), G> = <E, lookup_bwd(G)> for every shard (the adjoint of a
    # linear map is its gradient), the shards' gradients stacked equal
    # torch's embedding gradient, and a hand case sums repeated ids.
    rng = np.random.default_rng(11)
    T, V, K = 37, 24, 5
    ids = rng.integers(0, V, size=T)
    emb = rng.standard_normal((V, K))
    g = rng.standard_normal((T, K))
    vi = V // n
    grads = []
    for i in range(n):
        sh = emb[i * vi:(i + 1) * vi]
        lhs = np.sum(O.vocab_parallel_embedding(ids, sh, i * vi) * g)
        gi = O.vocab_parallel_embedding_bwd(ids, g, vi, i * vi)
        assert abs(lhs - np.sum(sh * gi)) <= 1e-12 * (1 + abs(lhs))
        grads.append(gi)
    e = torch.tensor(emb, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.embedding(torch.tensor(ids), e).backward(torch.tensor(g))
    assert np.allclose(np.concatenate(grads), e.grad.numpy(), rtol=0, atol=1e-12)
    hand = O.vocab_parallel_embedding_bwd([2, 0, 2, 5], np.array([[1.0], [10.0], [100.0], [7.0]]), 4, 0)
    assert np.array_equal(hand[:, 0], [10.0, 0.0, 101.0, 0.0])


def test_cross_entropy_matches_torch_and_closed_forms():
    z = rnd(17, 50) * 3
    y = RNG.integers(0, 50, size=17)
    ref = tF.cross_entropy(torch.tensor(z), torch.tensor(y), reduction="none").numpy()
    assert np.allclose(O.full_cross_entropy(z, y), ref, rtol=1e-13, atol=1e-13)
    # Zero logits: loss = ln V exactly; shift invariance; a dominant label -> ~0.
    assert np.allclose(O.full_cross_entropy(np.zeros((3, 51200)), [0, 7, 51199]), math.log(51200), atol=1e-12)
    assert np.allclose(O.full_cross_entropy(z + 123.0, y), O.full_cross_entropy(z, y), atol=1e-11)
    zd = z.copy()
    zd[np.arange(17), y] = 200.0
    assert np.all(O.full_cross_entropy(zd, y) < 1e-70 + 1e-12)


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_triples_combine_equals_full(n):
    t, v = 23, 96
    z = rnd(t, v) * 2
    y = RNG.integers(0, v, size=t)
    vi = v // n
    trip = [O.vocab_parallel_xent_triples(z[:, i * vi:(i + 1) * vi], y, i * vi) for i in range(n)]
    loss, big_m, big_s = O.vocab_xent_combine(trip)
    assert np.allclose(loss, O.full_cross_entropy(z, y), rtol=1e-13, atol=1e-13)
    assert np.allclose(big_m, z.max(axis=1))
    assert np.allclose(big_s, np.exp(z - big_m[:, None]).sum(axis=1), rtol=1e-13)
    # Exactly one shard owns each label.
    owners = sum((np.asarray([tr[:, 2] for tr in trip]) != 0).astype(int))
    assert np.all(owners <= 1)
    g = 1.0 / t
    grads = [O.vocab_parallel_xent_bwd(z[:, i * vi:(i + 1) * vi], y, i * vi, big_m, big_s, g) for i in range(n)]
    zt = torch.tensor(z, requires_grad=True)
    tF.cross_entropy(zt, torch.tensor(y), reduction="mean").backward()
    assert np.allclose(np.concatenate(grads, axis=1), zt.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert np.allclose(O.full_cross_entropy_grad(z, y, g), zt.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_triples_brute_force():
    z = rnd(3, 7)
    y = np.array([1, 9, 4])
    tr = O.vocab_parallel_xent_triples(z, y, 3)
    for r in range(3):
        m = max(z[r])
        assert tr[r, 0] == m
        assert abs(tr[r, 1] - sum(math.exp(val - m) for val in z[r])) < 1e-14
        assert tr[r, 2] == (z[r, y[r] - 3] if 3 <= y[r] < 10 else 0.0)


# ------------------------------------------------------------------ MoE

def routing(tokens, experts, topk):
    ids = np.stack([RNG.permutation(experts)[:topk] for _ in range(tokens)])
    w = RNG.random((tokens, topk))
    return ids, w / w.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("e_start,e_local", [(0, 4), (4, 4), (2, 3), (0, 16)])
def test_permutation_matches_stable_argsort(e_start, e_local):
    ids, _ = routing(50, 16, 4)
    counts, offsets, picks = O.moe_permutation(ids, e_start, e_local)
    flat = ids.reshape(-1)
    local = np.nonzero((flat >= e_start) & (flat < e_start + e_local))[0]
    order = local[np.argsort(flat[local], kind="stable")]
    assert np.array_equal(picks, order)
    assert counts.sum() == local.size
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(counts, np.bincount(flat[local] - e_start, minlength=e_local))


def test_expert_ffn_scalar_closed_form():
    # Hd = Fe = 1, gate weight 1, up weight 2, down weight 3, x = 1:
    # y = 3 * silu(1) * 2 with silu(1) = 1 / (1 + e^-1).
    y = O.expert_swiglu_ffn(np.array([[1.0]]), np.array([[1.0], [2.0]]), np.array([[3.0]]))
    assert abs(y[0, 0] - 6.0 / (1.0 + math.exp(-1.0))) < 1e-15


def test_expert_ffn_brute_force():
    hd, fe, r = 4, 3, 2
    x, wgu, wd = rnd(r, hd), rnd(2 * fe, hd), rnd(hd, fe)
    y = O.expert_swiglu_ffn(x, wgu, wd)
    for i in range(r):
        act = []
        for j in range(fe):
            g = sum(x[i, k] * wgu[j, k] for k in range(hd))
            u = sum(x[i, k] * wgu[fe + j, k] for k in range(hd))
            act.append(g / (1 + math.exp(-g)) * u)
        for o in range(hd):
            assert abs(y[i, o] - sum(act[j] * wd[o, j] for j in range(fe))) < 1e-13


def test_moe_forward_matches_per_token_definition():
    t, hd, fe, experts, topk, e_start, e_local = 30, 6, 5, 12, 3, 4, 4
    ids, w = routing(t, experts, topk)
    x = rnd(t, hd)
    wgu, wd = rnd(e_local, 2 * fe, hd, scale=0.5), rnd(e_local, hd, fe, scale=0.5)
    out, counts, offsets, picks, y_perm = O.moe_forward(x, ids, w, wgu, wd, e_start)
    ref = O.moe_forward_rows(x, ids, w, wgu, wd, e_start, list(range(t)))
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-14)
    none_local = ~np.any((ids >= e_start) & (ids < e_start + e_local), axis=1)
    assert np.all(out[none_local] == 0)
    # Linearity in the routing weights: doubling every weight doubles the output.
    out2 = O.moe_forward(x, ids, 2 * w, wgu, wd, e_start)[0]
    assert np.allclose(out2, 2 * out, rtol=1e-14, atol=1e-14)


def test_weighted_activation_form_equals_weighted_unpermute():
    """The memory-efficient form (weight on the activation, MOE-core 2.2)
    against the weighted-unpermute form and the per-token definition: equal in
    exact arithmetic because the down projection is linear; row by row its
    permuted output is the weight times the plain expert output."""
    t, hd, fe, experts, topk, e_start, e_local = 40, 7, 6, 10, 3, 2, 5
    ids, w = routing(t, experts, topk)
    x = rnd(t, hd)
    wgu, wd = rnd(e_local, 2 * fe, hd, scale=0.5), rnd(e_local, hd, fe, scale=0.5)
    out, counts, offsets, picks, y_perm = O.moe_forward_weighted_act(x, ids, w, wgu, wd, e_start)
    out_std, counts_std, offsets_std, picks_std, y_std = O.moe_forward(x, ids, w, wgu, wd, e_start)
    assert np.array_equal(picks, picks_std) and np.array_equal(offsets, offsets_std)
    assert np.allclose(out, out_std, rtol=1e-12, atol=1e-13)
    ref = O.moe_forward_rows(x, ids, w, wgu, wd, e_start, list(range(t)))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
    wflat = np.asarray(w, dtype=np.float64).reshape(-1)
    assert np.allclose(y_perm, wflat[picks][:, None] * y_std, rtol=1e-12, atol=1e-13)
    # Unit weights: both forms are the same computation.
    ones = np.ones_like(np.asarray(w, dtype=np.float64))
    assert np.allclose(O.moe_forward_weighted_act(x, ids, ones, wgu, wd, e_start)[4],
                       O.moe_forward(x, ids, ones, wgu, wd, e_start)[4], rtol=1e-13, atol=1e-14)
    # A token whose picks all land elsewhere gets zeros.
    none_local = ~np.any((ids >= e_start) & (ids < e_start + e_local), axis=1)
    assert np.all(out[none_local] == 0)


def _moe_loss(x, ids, w, wgu, wd, e_start, dout):
    """sum(dout * out) with out from the per-token definition (not the
    permuted code the backward mirrors)."""
    out = O.moe_forward_rows(x, ids, w, wgu, wd, e_start, list(range(x.shape[0])))
    return float(np.sum(dout * out))


def test_moe_backward_central_differences():
    """Every gradient of the MoE shard (input, gate/up and down weights,
    routing weights) against central finite differences of the per-token
    forward definition, at a tiny shape that includes a token with no local
    pick and a local expert nobody picks."""
    t, hd, fe, topk, e_start, e_local = 7, 5, 4, 2, 2, 4
    # Experts 2..5 are local; token 0 picks none of them and nobody picks
    # expert 5 (local index 3); ids are distinct per token.
    ids = np.array([[0, 7], [6, 1], [2, 6], [3, 2], [4, 0], [2, 4], [3, 1]])
    w = np.random.default_rng(77).random((t, topk))
    w = w / w.sum(axis=1, keepdims=True)
    x = rnd(t, hd)
    wgu, wd = rnd(e_local, 2 * fe, hd, scale=0.5), rnd(e_local, hd, fe, scale=0.5)
    dout = rnd(t, hd)
    g = O.moe_backward(x, ids, w, wgu, wd, e_start, dout)
    args = {"x": x, "w_gu": wgu, "w_d": wd, "topk_w": w}
    h = 1e-6
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _moe_loss(args["x"], ids, args["topk_w"], args["w_gu"], args["w_d"], e_start, dout)
            arr[idx] = keep - h
            lm = _moe_loss(args["x"], ids, args["topk_w"], args["w_gu"], args["w_d"], e_start, dout)
            arr[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(g[name] - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err <= 1e-6, (name, err)
    assert np.all(g["x"][0] == 0) and np.all(g["topk_w"][0] == 0)
    assert np.all(g["w_gu"][3] == 0) and np.all(g["w_d"][3] == 0)
    local = (ids >= e_start) & (ids < e_start + e_local)
    assert np.all(g["topk_w"][~local] == 0)


def test_moe_backward_matches_torch_autograd():
    """The same gradients from torch's float64 autograd through a per-token
    forward written with torch ops (an independent library routine)."""
    t, hd, fe, experts, topk, e_start, e_local = 40, 12, 10, 16, 4, 4, 6
    ids, w = routing(t, experts, topk)
    x = rnd(t, hd)
    wgu, wd = rnd(e_local, 2 * fe, hd, scale=0.3), rnd(e_local, hd, fe, scale=0.3)
    dout = rnd(t, hd)
    g = O.moe_backward(x, ids, w, wgu, wd, e_start, dout)
    tx, tw = torch.tensor(x, requires_grad=True), torch.tensor(w, requires_grad=True)
    tgu, td = torch.tensor(wgu, requires_grad=True), torch.tensor(wd, requires_grad=True)
    rows = []
    for i in range(t):
        acc = torch.zeros(hd, dtype=torch.float64)
        for k in range(topk):
            e = int(ids[i, k]) - e_start
            if 0 <= e < e_local:
                act = tF.silu(tgu[e, :fe] @ tx[i]) * (tgu[e, fe:] @ tx[i])
                acc = acc + tw[i, k] * (td[e] @ act)
        rows.append(acc)
    (torch.stack(rows) * torch.tensor(dout)).sum().backward()
    for name, ref in (("x", tx), ("topk_w", tw), ("w_gu", tgu), ("w_d", td)):
        r = ref.grad.numpy()
        assert np.allclose(g[name], r, rtol=1e-11, atol=1e-12), name


def _moe_loss_weighted_act(x, ids, w, wgu, wd, e_start, dout):
    """sum(dout * out) through the memory-efficient form's forward."""
    return float(np.sum(dout * O.moe_forward_weighted_act(x, ids, w, wgu, wd, e_start)[0]))


def test_moe_backward_weighted_act_central_differences():
    """The memory-efficient form's backward against central finite
    differences of its own forward, and against the weighted-unpermute
    form's backward (the same function, so the same gradients)."""
    t, hd, fe, topk, e_start, e_local = 7, 5, 4, 2, 2, 4
    ids = np.array([[0, 7], [6, 1], [2, 6], [3, 2], [4, 0], [2, 4], [3, 1]])
    w = np.random.default_rng(78).random((t, topk))
    w = w / w.sum(axis=1, keepdims=True)
    rng = np.random.default_rng(79)
    x = rng.standard_normal((t, hd))
    wgu, wd = rng.standard_normal((e_local, 2 * fe, hd)) * 0.5, rng.standard_normal((e_local, hd, fe)) * 0.5
    dout = rng.standard_normal((t, hd))
    g = O.moe_backward_weighted_act(x, ids, w, wgu, wd, e_start, dout)
    args = {"x": x, "w_gu": wgu, "w_d": wd, "topk_w": w}
    h = 1e-6
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _moe_loss_weighted_act(args["x"], ids, args["topk_w"], args["w_gu"], args["w_d"], e_start, dout)
            arr[idx] = keep - h
            lm = _moe_loss_weighted_act(args["x"], ids, args["topk_w"], args["w_gu"], args["w_d"], e_start, dout)
            arr[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(g[name] - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err <= 1e-6, (name, err)
    std = O.moe_backward(x, ids, w, wgu, wd, e_start, dout)
    for name in args:
        assert np.allclose(g[name], std[name], rtol=1e-11, atol=1e-13), name
