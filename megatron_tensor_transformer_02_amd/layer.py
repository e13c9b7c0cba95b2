"""One tensor-parallel rank's share of a transformer layer, driven through libmp.

Orchestration only: every step is a libmp call (see :mod:`.mp`); this module
owns the device buffers and the order of the calls.  The stages are split at
each reduce (the all-reduce of the pages, MLM-notes "Model Parallel
Transformers": one all-reduce after the attention block and one after the
MLP in the forward, two in the backward), so N ranks can be emulated on one
GPU: run every rank's ``*_partial`` stage, then feed all partials to one
rank's ``*_reduce`` stage, which calls ``mp_shard_reduce`` or, where a
LayerNorm follows the reduce, the fused ``mp_shard_reduce_layernorm`` /
``mp_shard_reduce_layernorm_bwd``.

Layer (pre-LN; the placement the GPT-2-style block uses):
``H1 = X + Drop(sum_i Attn_i(LN1(X)) W_o,i^T + b_o)``,
``Out = H1 + Drop(sum_i GeLU(LN2(H1) A_i^T + a_i) B_i^T + b_b)``.
"""

import torch

from . import mp


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


class RankLayer:
    """Rank ``i``'s layer share.  ``shard`` holds this rank's ``w_qkv, b_qkv,
    w_o, w_a, b_a, w_b`` (contiguous device tensors, as cut by
    ``synthetic.rank_shard``); ``shared`` the replicated ``ln1_g, ln1_b,
    ln2_g, ln2_b, b_o, b_b``."""

    def __init__(self, shard, shared, B, L, heads, d, p=0.1, seed=0, offsets=(1, 2), eps=1e-5, act="erf",
                 causal=True):
        self.s, self.c = shard, shared
        self.B, self.L, self.nh, self.d = B, L, heads, d
        self.p, self.seed, self.off = p, seed, offsets
        self.eps, self.act, self.causal = eps, act, causal
        # Optional callable(tag) invoked right before and after the
        # column-parallel GEMM (tags "col_begin", "col_end"), e.g. to record
        # timing events around that one kernel.
        self.probe = None
        dev = shard["w_qkv"].device
        dt = shard["w_qkv"].dtype
        T = B * L
        K = shard["w_qkv"].shape[1]
        Fi = shard["w_a"].shape[0]
        hd = heads * d
        self.T, self.K, self.Fi = T, K, Fi
        f32 = torch.float32
        e = lambda *shape: _empty(shape, dt, dev)  # noqa: E731
        # forward activations
        self.h, self.qkv, self.ctx = e(T, K), e(T, 3 * hd), e(T, hd)
        self.mu1, self.rs1 = _empty(T, f32, dev), _empty(T, f32, dev)
        self.lse = _empty((B, heads, L), f32, dev)
        self.p_attn, self.h1, self.h2, self.p_mlp, self.out = e(T, K), e(T, K), e(T, K), e(T, K), e(T, K)
        self.mu2, self.rs2 = _empty(T, f32, dev), _empty(T, f32, dev)
        self.y, self.z = e(T, Fi), e(T, Fi)
        # keep flags of the two dropouts, one bit per element, for the backward
        self.keep_attn = _empty(((T * K + 7) // 8,), torch.uint8, dev)
        self.keep_mlp = _empty(((T * K + 7) // 8,), torch.uint8, dev)
        # backward buffers
        self.d_mlp, self.dy, self.dh2p, self.dh1 = e(T, K), e(T, Fi), e(T, K), e(T, K)
        self.d_attn, self.dctx, self.dhp, self.dx = e(T, K), e(T, hd), e(T, K), e(T, K)
        self.g = {
            "w_qkv": _empty(shard["w_qkv"].shape, f32, dev), "b_qkv": _empty(shard["b_qkv"].shape, f32, dev),
            "w_o": _empty(shard["w_o"].shape, f32, dev), "b_o": _empty(K, f32, dev),
            "w_a": _empty(shard["w_a"].shape, f32, dev), "b_a": _empty(Fi, f32, dev),
            "w_b": _empty(shard["w_b"].shape, f32, dev), "b_b": _empty(K, f32, dev),
            "ln1_g": _empty(K, f32, dev), "ln1_b": _empty(K, f32, dev),
            "ln2_g": _empty(K, f32, dev), "ln2_b": _empty(K, f32, dev),
        }

    # ------------------------------------------------------------ forward
    def attn_partial(self, x):
        s, c = self.s, self.c
        mp.mp_layernorm(x, c["ln1_g"], c["ln1_b"], self.h, self.mu1, self.rs1, self.eps)
        mp.mp_head_attention(self.h, s["w_qkv"], s["b_qkv"], self.B, self.L, self.nh, self.d, self.ctx,
                             self.qkv, self.lse, self.causal)
        mp.mp_row_linear_partial(self.ctx, s["w_o"], self.p_attn)
        return self.p_attn

    def attn_reduce(self, partials, x):
        # The reduce and the LN2 it feeds in one pass: H1 and LN2(H1).
        c = self.c
        mp.mp_shard_reduce_layernorm(partials, self.h1, c["ln2_g"], c["ln2_b"], self.h2, self.mu2, self.rs2,
                                     bias=c["b_o"], residual=x, p=self.p, seed=self.seed, offset=self.off[0],
                                     mask_out=self.keep_attn, eps=self.eps)
        return self.h1

    def mlp_partial(self):
        s = self.s
        if self.probe is not None:
            self.probe("col_begin")
        mp.mp_column_linear_gelu(self.h2, s["w_a"], s["b_a"], self.act, self.y, self.z)
        if self.probe is not None:
            self.probe("col_end")
        mp.mp_row_linear_partial(self.y, s["w_b"], self.p_mlp)
        return self.p_mlp

    def mlp_reduce(self, partials):
        mp.mp_shard_reduce(partials, self.out, self.c["b_b"], self.h1, self.p, self.seed, self.off[1], 0,
                           self.keep_mlp)
        return self.out

    # ----------------------------------------------------------- backward
    def mlp_bwd_partial(self, dout):
        s, g = self.s, self.g
        # Dropout backward from the saved keep bits, with the bias gradient.
        mp.mp_dropout_mask_bwd(dout, self.keep_mlp, self.p, self.d_mlp, g["b_b"])
        # The GeLU gradient is applied in the epilogue of the row-parallel
        # input-gradient GEMM, so the column backward gets dZ directly.
        mp.mp_row_linear_partial_bwd_dact(self.y, s["w_b"], self.d_mlp, self.z, self.act, self.dy, g["w_b"])
        mp.mp_column_linear_gelu_bwd(self.h2, s["w_a"], None, self.dy, "none", self.dh2p, g["w_a"], g["b_a"])
        return self.dh2p

    def mlp_bwd_reduce(self, partials, dout):
        # Backward all-reduce of the MLP input gradient fused with LN2's
        # backward; the residual branch adds dOut.  The same pass starts the
        # attention block's backward: its output dropout (the keep bits saved
        # by the forward) applied to dH1 and the column sums of the result
        # (the out-projection bias gradient).
        c, g = self.c, self.g
        mp.mp_shard_reduce_layernorm_bwd_dropout(partials, self.h1, c["ln2_g"], self.mu2, self.rs2, self.dh1, self.p,
                                                 self.keep_attn, self.d_attn, dres=dout, dgamma=g["ln2_g"],
                                                 dbeta=g["ln2_b"], dbias=g["b_o"])
        return self.dh1

    def attn_bwd_partial(self):
        s, g = self.s, self.g
        mp.mp_row_linear_partial_bwd(self.ctx, s["w_o"], self.d_attn, self.dctx, g["w_o"])
        mp.mp_head_attention_bwd(self.h, s["w_qkv"], self.qkv, self.ctx, self.lse, self.dctx, self.B, self.L,
                                 self.nh, self.d, self.dhp, g["w_qkv"], g["b_qkv"], self.causal)
        return self.dhp

    def attn_bwd_reduce(self, partials, x):
        c, g = self.c, self.g
        mp.mp_shard_reduce_layernorm_bwd(partials, x, c["ln1_g"], self.mu1, self.rs1, self.dx, self.dh1, g["ln1_g"],
                                         g["ln1_b"])
        return self.dx


def make_ranks(shards, shared, B, L, heads_per_rank, d, **kw):
    ranks = []
    for sh in shards:
        ranks.append(RankLayer(sh, shared, B, L, heads_per_rank, d, **kw))
    return ranks


def run_ranks(ranks, x, dout):
    """Emulates N ranks on one GPU (every rank's stages, with the shard reduce
    standing in for each all-reduce).  Returns every stage's partials so a
    single rank can later be replayed against them."""
    pa = [r.attn_partial(x) for r in ranks]
    for r in ranks:
        r.attn_reduce(pa, x)
    pm = [r.mlp_partial() for r in ranks]
    for r in ranks:
        r.mlp_reduce(pm)
    pb = [r.mlp_bwd_partial(dout) for r in ranks]
    for r in ranks:
        r.mlp_bwd_reduce(pb, dout)
    pq = [r.attn_bwd_partial() for r in ranks]
    for r in ranks:
        r.attn_bwd_reduce(pq, x)
    return {"attn": pa, "mlp": pm, "mlp_bwd": pb, "attn_bwd": pq}


class VocabShard:
    """Rank ``i``'s vocab shard: embedding rows ``E_i = E[v_start : v_start+Vi]``
    used both for the input lookup and the output logits (tied weights)."""

    def __init__(self, E_i, v_start, T):
        self.E, self.v0 = E_i, v_start
        dev = E_i.device
        Vi, K = E_i.shape
        self.emb = torch.empty((T, K), dtype=E_i.dtype, device=dev)
        self.emb_sum = torch.empty((T, K), dtype=E_i.dtype, device=dev)
        self.z = torch.empty((T, Vi), dtype=torch.float32, device=dev)
        self.tr = torch.empty((T, 3), dtype=torch.float32, device=dev)
        self.loss = torch.empty(T, dtype=torch.float32, device=dev)
        self.stats = torch.empty((T, 2), dtype=torch.float32, device=dev)
        self.mean = torch.empty(1, dtype=torch.float32, device=dev)

    def embed_partial(self, ids):
        mp.mp_vocab_parallel_embedding(ids, self.E, self.v0, self.emb)
        return self.emb

    def embed_reduce(self, partials):
        mp.mp_shard_reduce(partials, self.emb_sum)
        return self.emb_sum

    def logits(self, hidden):
        mp.mp_column_linear_gelu(hidden, self.E, None, "none", self.z)
        return self.z

    def triples(self, labels):
        mp.mp_vocab_parallel_xent(self.z, labels, self.v0, self.tr)
        return self.tr

    def combine(self, triples):
        mp.mp_vocab_xent_combine(triples, self.loss, self.stats, self.mean)
        return self.loss

    def xent_bwd(self, labels, g):
        mp.mp_vocab_parallel_xent_bwd(self.z, labels, self.v0, self.stats, g, self.z)
        return self.z
