"""Oracle of the vocab-parallel embedding and cross-entropy (fp64).

Test infrastructure only (see the package docstring).  MLM-notes, "Model
Parallel Transformers", embedding paragraph: the ``V x K`` embedding is split,
``X`` is replicated, each side looks up, then an all-reduce.  Output paragraph:
the ``B x L x V`` logits are sharded over V; each GPU computes its
exponentials first and the row-wise sums are combined.

Readings: the split is along V (a rank owns whole rows ``[v_start,
v_start + V_i)`` and contributes zeros for ids it does not own, the only split
for which "look up, then all-reduce" sums correctly); each shard reports a row
maximum as well as its exp-sum so the combine is numerically safe; the loss
is per token with no ignore index, and its mean over tokens is also reported.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def embedding(ids, emb):
    """Full lookup ``E[id]`` for every token."""
    return _f64(emb)[np.asarray(ids, dtype=np.int64)]


def vocab_parallel_embedding(ids, emb_shard, v_start):
    """One rank's partial lookup: row ``id - v_start`` of its shard where the
    id is owned, zeros elsewhere."""
    ids = np.asarray(ids, dtype=np.int64)
    emb_shard = _f64(emb_shard)
    out = np.zeros((ids.size, emb_shard.shape[1]))
    own = (ids >= v_start) & (ids < v_start + emb_shard.shape[0])
    out[own] = emb_shard[ids[own] - v_start]
    return out


def vocab_parallel_embedding_bwd(ids, d_out, vi, v_start):
    """Gradient of one rank's partial lookup with respect to its shard: the
    lookup copies row ``id - v_start`` into token t's output, so row v of the
    gradient is the sum of ``d_out[t]`` over the tokens t whose id is
    ``v_start + v`` (zero for rows no token picked).  Summed token by token in
    ascending order."""
    ids = np.asarray(ids, dtype=np.int64)
    d_out = _f64(d_out)
    grad = np.zeros((vi, d_out.shape[1]))
    for t in range(ids.size):
        v = ids[t] - v_start
        if 0 <= v < vi:
            grad[v] += d_out[t]
    return grad


def full_cross_entropy(logits, labels):
    """Per-token softmax cross-entropy over the full vocabulary:
    ``log(sum_v exp(z_v)) - z_label``, the max subtracted inside the log."""
    z = _f64(logits)
    labels = np.asarray(labels, dtype=np.int64)
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return lse - z[np.arange(z.shape[0]), labels]


def full_cross_entropy_grad(logits, labels, g):
    """``d loss_total / d z = g * (softmax(z) - onehot(label))``."""
    z = _f64(logits)
    labels = np.asarray(labels, dtype=np.int64)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    grad = e / e.sum(axis=1, keepdims=True)
    grad[np.arange(z.shape[0]), labels] -= 1.0
    return g * grad


def vocab_parallel_xent_triples(z_shard, labels, v_start):
    """Per-row statistics of one vocab shard ``Z_i [T, V_i]``:
    ``m = max_v z``, ``s = sum_v exp(z - m)``, ``t = z[label - v_start]`` if
    the label is owned by this shard, else 0.  Returns ``[T, 3]``."""
    z = _f64(z_shard)
    labels = np.asarray(labels, dtype=np.int64)
    m = z.max(axis=1)
    s = np.exp(z - m[:, None]).sum(axis=1)
    t = np.zeros(z.shape[0])
    own = (labels >= v_start) & (labels < v_start + z.shape[1])
    rows = np.nonzero(own)[0]
    t[rows] = z[rows, labels[rows] - v_start]
    return np.stack([m, s, t], axis=1)


def vocab_xent_combine(triples):
    """Combine the shards' row statistics (the row-wise sums combined across
    GPUs): ``M = max_j m_j``, ``S = sum_j s_j exp(m_j - M)``,
    ``loss = log S + M - sum_j t_j``.  Returns ``(loss [T], M [T], S [T])``."""
    tr = [_f64(x) for x in triples]
    big_m = np.max(np.stack([x[:, 0] for x in tr]), axis=0)
    big_s = np.zeros_like(big_m)
    tgt = np.zeros_like(big_m)
    for x in tr:
        big_s = big_s + x[:, 1] * np.exp(x[:, 0] - big_m)
        tgt = tgt + x[:, 2]
    return np.log(big_s) + big_m - tgt, big_m, big_s


def vocab_parallel_xent_bwd(z_shard, labels, v_start, big_m, big_s, g):
    """One shard's logits gradient ``g * (exp(z - M) / S - [v_start + col == label])``."""
    z = _f64(z_shard)
    labels = np.asarray(labels, dtype=np.int64)
    grad = np.exp(z - _f64(big_m)[:, None]) / _f64(big_s)[:, None]
    own = (labels >= v_start) & (labels < v_start + z.shape[1])
    rows = np.nonzero(own)[0]
    grad[rows, labels[rows] - v_start] -= 1.0
    return g * grad
