"""Seeded synthetic inputs for the five workloads of the tensor-parallel shard.

This module only draws inputs: it holds none of the layer's arithmetic and is
shared, unchanged, by the parity tests (which feed both the HIP library and
the CPU oracle), ``bench.py`` and the smoke test.  Every tensor comes from
``numpy.random.default_rng(SeedSequence([workload_seed, tensor_id]))``; bf16
workloads round float32 draws to bfloat16 (round-to-nearest-even) with torch
on the CPU.  Tensors are returned as CPU torch tensors.

Workloads (sizes of the pages' models: MLM-notes "Model Parallel Transformers"
for the split, MLM-review "results" for the 8.3B GPT-2-like model, MOE-core
"technical summary" for the MoE shard):

* ``tiny``   -- MLP + vocab cross-entropy split N=2 in fp32: B=2, L=16, K=64,
  FFN 256 (two shards of 128), V=128 (two shards of 64), dropout p=0.1.
* ``gpt2m``  -- GPT-2-medium-shaped full layer at N=1 in bf16: K=1024,
  16 heads of 64, FFN 4096, causal, L=1024, B=8.
* ``mlm8b``  -- one rank's share of the 8.3B-config layer at N=8 in bf16:
  K=3072, 3 of 24 heads of 128, FFN shard 12288/8, L=1024, B=8.
* ``vocab``  -- vocab-parallel embedding + cross-entropy, one shard of N=8:
  V=51200 (6400 rows per shard), K=3072, 8x1024 tokens.
* ``moe``    -- expert shard: 8 local experts of 256, hidden 7168, expert FFN
  2048 (SwiGLU), 4096 tokens with top-8 routing, Zipf(1.1) popularity.
"""

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str                 # "f32" or "bf16"
    B: int = 0
    L: int = 0
    K: int = 0
    heads: int = 0
    d: int = 0
    F: int = 0
    N: int = 1
    V: int = 0
    p: float = 0.1
    T_moe: int = 0
    Fe: int = 0
    experts: int = 0
    e_local: int = 0
    topk: int = 0
    zipf: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.T_moe if self.T_moe else self.B * self.L


WORKLOADS = {
    "tiny": Workload("tiny", 101, "f32", B=2, L=16, K=64, F=256, N=2, V=128, p=0.1),
    "gpt2m": Workload("gpt2m", 202, "bf16", B=8, L=1024, K=1024, heads=16, d=64, F=4096, N=1, p=0.1),
    "mlm8b": Workload("mlm8b", 303, "bf16", B=8, L=1024, K=3072, heads=24, d=128, F=12288, N=8, p=0.1),
    "vocab": Workload("vocab", 404, "bf16", B=8, L=1024, K=3072, V=51200, N=8),
    "moe": Workload("moe", 505, "bf16", K=7168, T_moe=4096, Fe=2048, experts=256, e_local=8,
                    topk=8, zipf=1.1),
}

# Stable tensor ids: one per named tensor, so adding a tensor never changes
# the draws of another.
_TENSOR_IDS = {name: i for i, name in enumerate([
    "x", "w_qkv", "b_qkv", "w_o", "b_o", "w_a", "b_a", "w_b", "b_b", "dout",
    "ln1_g", "ln1_b", "ln2_g", "ln2_b", "labels", "emb", "hidden", "ids",
    "route_gumbel", "route_logits", "w_gu", "w_d", "moe_x", "dlogits",
])}


def rng_for(seed, tensor, salt=0):
    return np.random.default_rng(np.random.SeedSequence([int(seed), _TENSOR_IDS[tensor], int(salt)]))


def to_dtype(a, dtype):
    """float32 numpy array -> CPU torch tensor of the workload dtype (RNE for bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def normal(seed, tensor, shape, std=1.0, dtype="f32", salt=0):
    a = rng_for(seed, tensor, salt).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_dtype(a, dtype)


def uniform_int(seed, tensor, shape, high, salt=0):
    a = rng_for(seed, tensor, salt).integers(0, high, size=shape, dtype=np.int64)
    return torch.from_numpy(a.astype(np.int32))


def as_f64(t):
    """Exact float64 numpy copy of a CPU/GPU torch tensor (bf16 widens exactly)."""
    return t.detach().to("cpu", torch.float64).numpy()


# --------------------------------------------------------------------------
# Dense layer tensors
# --------------------------------------------------------------------------

def layer_params(wl, heads=None, d=None, K=None, F=None, std=0.02):
    """Full (unpartitioned) weights of one layer, ``[out, in]`` row-major.
    The fused QKV weight holds Q rows of all heads, then K rows, then V rows.
    LayerNorm gamma = 1 and beta = 0."""
    heads = heads or wl.heads
    d = d or wl.d
    K = K or wl.K
    F = F or wl.F
    hd = heads * d
    s, dt = wl.seed, wl.dtype
    one = to_dtype(np.ones(K, np.float32), dt)
    zero = to_dtype(np.zeros(K, np.float32), dt)
    return {
        "w_qkv": normal(s, "w_qkv", (3 * hd, K), std, dt), "b_qkv": normal(s, "b_qkv", (3 * hd,), std, dt),
        "w_o": normal(s, "w_o", (K, hd), std, dt), "b_o": normal(s, "b_o", (K,), std, dt),
        "w_a": normal(s, "w_a", (F, K), std, dt), "b_a": normal(s, "b_a", (F,), std, dt),
        "w_b": normal(s, "w_b", (K, F), std, dt), "b_b": normal(s, "b_b", (K,), std, dt),
        "ln1_g": one, "ln1_b": zero, "ln2_g": one.clone(), "ln2_b": zero.clone(),
    }


def layer_activations(wl, T=None, K=None):
    T = T or wl.T
    K = K or wl.K
    return (normal(wl.seed, "x", (T, K), 1.0, wl.dtype),
            normal(wl.seed, "dout", (T, K), 1.0, wl.dtype))


def rank_shard(prm, rank, n, heads, d):
    """Rank ``rank`` of ``n``: its heads' rows of the fused QKV weight (Q, K, V
    blocks kept in that order), the matching columns of ``w_o``, rows of
    ``w_a``/``b_a`` and columns of ``w_b``, each as a contiguous tensor.  The
    replicated biases ``b_o``/``b_b`` and LayerNorm parameters are shared.
    ``n`` must divide the head count and the FFN width (MLM-notes, "Model
    Parallel Transformers": the GPU count has to divide the attention heads);
    a remainder raises ValueError."""
    F = prm["w_a"].shape[0]
    if n < 1 or not 0 <= rank < n:
        raise ValueError(f"rank {rank} of {n} ranks")
    if heads % n:
        raise ValueError(f"{n} ranks do not divide {heads} attention heads")
    if F % n:
        raise ValueError(f"{n} ranks do not divide the FFN width {F}")
    hi = heads // n
    hd = heads * d
    rows = []
    for blk in range(3):
        rows.append(torch.arange(blk * hd + rank * hi * d, blk * hd + (rank + 1) * hi * d))
    rows = torch.cat(rows)
    fi = F // n
    fs = slice(rank * fi, (rank + 1) * fi)
    cs = slice(rank * hi * d, (rank + 1) * hi * d)
    return {
        "w_qkv": prm["w_qkv"][rows].contiguous(), "b_qkv": prm["b_qkv"][rows].contiguous(),
        "w_o": prm["w_o"][:, cs].contiguous(),
        "w_a": prm["w_a"][fs].contiguous(), "b_a": prm["b_a"][fs].contiguous(),
        "w_b": prm["w_b"][:, fs].contiguous(),
        "heads": hi,
    }


# --------------------------------------------------------------------------
# Vocab tensors
# --------------------------------------------------------------------------

def vocab_shard_rows(V, n):
    """Rows of each of ``n`` vocabulary shards; ``n`` must divide ``V``."""
    if n < 1 or V % n:
        raise ValueError(f"{n} ranks do not divide the vocabulary of {V}")
    return V // n


def vocab_inputs(wl, T=None, V=None, K=None, std=0.02):
    """Embedding ``[V, K]`` (~N(0, std)), hidden states ``[T, K]`` (~N(0,1)),
    token ids and labels uniform over the full vocabulary."""
    T = T or wl.T
    V = V or wl.V
    K = K or wl.K
    return {
        "emb": normal(wl.seed, "emb", (V, K), std, wl.dtype),
        "hidden": normal(wl.seed, "hidden", (T, K), 1.0, wl.dtype),
        "ids": uniform_int(wl.seed, "ids", (T,), V),
        "labels": uniform_int(wl.seed, "labels", (T,), V),
    }


# --------------------------------------------------------------------------
# MoE routing and expert weights
# --------------------------------------------------------------------------

def zipf_topk_routing(seed, tokens, experts, topk, s):
    """Top-k distinct expert ids per token, drawn without replacement with
    probability proportional to ``(e + 1) ** -s`` (Gumbel-top-k), in
    descending key order, plus routing weights: a softmax over the k picks of
    N(0,1) logits (they sum to one over all k picks, local or not)."""
    logp = -s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    g = rng_for(seed, "route_gumbel").gumbel(size=(tokens, experts))
    key = logp[None, :] + g
    ids = np.argsort(-key, axis=1, kind="stable")[:, :topk]
    lg = rng_for(seed, "route_logits").standard_normal(size=(tokens, topk))
    w = np.exp(lg - lg.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return (torch.from_numpy(ids.astype(np.int32)),
            torch.from_numpy(w.astype(np.float32)))


def moe_inputs(wl, T=None, Hd=None, Fe=None, e_local=None, e_start=0, std=0.02):
    """Hidden states ``[T, Hd]``, routing over ``wl.experts`` experts, and the
    weights of the local experts ``e_start .. e_start + e_local - 1``:
    ``w_gu [e_local, 2*Fe, Hd]`` (gate rows, then up rows) and
    ``w_d [e_local, Hd, Fe]``."""
    T = T or wl.T
    Hd = Hd or wl.K
    Fe = Fe or wl.Fe
    e_local = e_local or wl.e_local
    ids, w = zipf_topk_routing(wl.seed, T, wl.experts, wl.topk, wl.zipf)
    w_gu = torch.stack([normal(wl.seed, "w_gu", (2 * Fe, Hd), std, wl.dtype, salt=e)
                        for e in range(e_start, e_start + e_local)])
    w_d = torch.stack([normal(wl.seed, "w_d", (Hd, Fe), std, wl.dtype, salt=e)
                       for e in range(e_start, e_start + e_local)])
    return {"x": normal(wl.seed, "moe_x", (T, Hd), 1.0, wl.dtype), "topk_ids": ids,
            "topk_w": w, "w_gu": w_gu, "w_d": w_d}
