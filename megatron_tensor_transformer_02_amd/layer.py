"""One tensor-parallel rank's share of a transformer layer, driven through libmp.

Orchestration only: every step is a libmp call (see :mod:`.mp`); this module
owns the device buffers and the order of the calls.  The stages are split at
each reduce (the all-reduce of the pages, MLM-notes "Model Parallel
Transformers": one all-reduce after the attention block and one after the
MLP in the forward, two in the backward), so N ranks can be emulated on one
GPU: run every rank's ``*_partial`` stage, then feed all partials to one
rank's ``*_reduce`` stage, which calls ``mp_shard_reduce`` or, where a
LayerNorm follows the reduce, the fused ``mp_shard_reduce_layernorm`` /
``mp_shard_reduce_layernorm_bwd``.  :class:`SPRankLayer` is the
sequence-parallel form (reduce-scatter and all-gather in place of each
all-reduce).

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
        c = self.c
        mp.mp_layernorm(x, c["ln1_g"], c["ln1_b"], self.h, self.mu1, self.rs1, self.eps)
        return self.attn_core()

    def attn_core(self):
        # Attention over this rank's heads of LN1(X) (in self.h), then the
        # out-projection's partial sum.
        s = self.s
        if self.probe is not None:
            self.probe("attn_fwd_begin")
        mp.mp_head_attention(self.h, s["w_qkv"], s["b_qkv"], self.B, self.L, self.nh, self.d, self.ctx,
                             self.qkv, self.lse, self.causal)
        if self.probe is not None:
            self.probe("attn_fwd_end")
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
        # Dropout backward from the saved keep bits, with the bias gradient.
        mp.mp_dropout_mask_bwd(dout, self.keep_mlp, self.p, self.d_mlp, self.g["b_b"])
        return self.mlp_bwd_core()

    def mlp_bwd_core(self):
        s, g = self.s, self.g
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
        if self.probe is not None:
            self.probe("attn_bwd_begin")
        mp.mp_head_attention_bwd(self.h, s["w_qkv"], self.qkv, self.ctx, self.lse, self.dctx, self.B, self.L,
                                 self.nh, self.d, self.dhp, g["w_qkv"], g["b_qkv"], self.causal)
        if self.probe is not None:
            self.probe("attn_bwd_end")
        return self.dhp

    def attn_bwd_reduce(self, partials, x):
        c, g = self.c, self.g
        mp.mp_shard_reduce_layernorm_bwd(partials, x, c["ln1_g"], self.mu1, self.rs1, self.dx, self.dh1, g["ln1_g"],
                                         g["ln1_b"])
        return self.dx


class SPRankLayer(RankLayer):
    """Rank ``r`` of ``n`` in the sequence-parallel form of the same layer
    (PAR-survey, "Achievement" item 4 and "How": TP+SP spreads LayerNorm,
    dropout and the residual over the ranks along the sequence; read here as
    each all-reduce becoming a reduce-scatter followed, before the next
    column-parallel GEMM, by an all-gather).  The rank owns tokens ``[r*T/n, (r+1)*T/n)`` for LayerNorm,
    dropout and the residual; its attention and MLP work on the gathered
    full sequence exactly as in :class:`RankLayer`.  The reduce-scatter is a
    shard reduce over the rank's rows of every partial, with the dropout
    drawn at the global element index; ``mp_all_gather_rows`` stands in for
    the all-gather.  The replicated parameters' gradients (LayerNorm, the two
    reduced biases) cover the rank's tokens only: the ranks' values sum to the
    full gradient (the all-reduce a real run would do)."""

    def __init__(self, shard, shared, B, L, heads, d, rank, n, **kw):
        super().__init__(shard, shared, B, L, heads, d, **kw)
        assert (B * L) % n == 0, "tokens must split evenly over the ranks"
        self.rank, self.n = rank, n
        self.ts = B * L // n
        self.r0, self.r1 = rank * self.ts, (rank + 1) * self.ts

    def _rows(self, t):
        return t[self.r0:self.r1]

    def _bits(self, keep):
        k = self.K
        return keep[self.r0 * k // 8:self.r1 * k // 8]

    # ------------------------------------------------------------ forward
    def ln1_slice(self, x_slice):
        c = self.c
        mp.mp_layernorm(x_slice, c["ln1_g"], c["ln1_b"], self._rows(self.h), self._rows(self.mu1),
                        self._rows(self.rs1), self.eps)

    def attn_reduce(self, partials, x_slice):
        # Reduce-scatter + bias + dropout + residual on the rank's tokens,
        # fused with LN2 of those tokens.
        c = self.c
        mp.mp_shard_reduce_layernorm([self._rows(p) for p in partials], self._rows(self.h1), c["ln2_g"], c["ln2_b"],
                                     self._rows(self.h2), self._rows(self.mu2), self._rows(self.rs2), bias=c["b_o"],
                                     residual=x_slice, p=self.p, seed=self.seed, offset=self.off[0],
                                     index_base=self.r0 * self.K, mask_out=self._bits(self.keep_attn), eps=self.eps)
        return self._rows(self.h1)

    def mlp_reduce(self, partials):
        mp.mp_shard_reduce([self._rows(p) for p in partials], self._rows(self.out), self.c["b_b"],
                           self._rows(self.h1), self.p, self.seed, self.off[1], self.r0 * self.K,
                           self._bits(self.keep_mlp))
        return self._rows(self.out)

    # ----------------------------------------------------------- backward
    def mlp_bwd_slice(self, dout_slice):
        mp.mp_dropout_mask_bwd(dout_slice, self._bits(self.keep_mlp), self.p, self._rows(self.d_mlp), self.g["b_b"])

    def mlp_bwd_reduce(self, partials, dout_slice):
        c, g = self.c, self.g
        mp.mp_shard_reduce_layernorm_bwd_dropout([self._rows(p) for p in partials], self._rows(self.h1), c["ln2_g"],
                                                 self._rows(self.mu2), self._rows(self.rs2), self._rows(self.dh1),
                                                 self.p, self._bits(self.keep_attn), self._rows(self.d_attn),
                                                 dres=dout_slice, dgamma=g["ln2_g"], dbeta=g["ln2_b"],
                                                 dbias=g["b_o"])
        return self._rows(self.dh1)

    def attn_bwd_reduce(self, partials, x_slice):
        c, g = self.c, self.g
        mp.mp_shard_reduce_layernorm_bwd([self._rows(p) for p in partials], x_slice, c["ln1_g"], self._rows(self.mu1),
                                         self._rows(self.rs1), self._rows(self.dx), self._rows(self.dh1),
                                         g["ln1_g"], g["ln1_b"])
        return self._rows(self.dx)


def gather(ranks, name):
    """The all-gather of every rank's slice of buffer ``name`` into each rank's
    full buffer (one ``mp_all_gather_rows`` per rank)."""
    slices = [r._rows(getattr(r, name)) for r in ranks]
    for r in ranks:
        mp.mp_all_gather_rows(slices, getattr(r, name))


def run_ranks_sp(ranks, x, dout):
    """Emulates the n sequence-parallel ranks on one GPU; ``x``, ``dout`` are
    the full [T, K] input and upstream gradient, of which rank r reads only
    its token slice.  Returns every stage's partials, as :func:`run_ranks`."""
    for r in ranks:
        r.ln1_slice(r._rows(x))
    gather(ranks, "h")
    pa = [r.attn_core() for r in ranks]
    for r in ranks:
        r.attn_reduce(pa, r._rows(x))
    gather(ranks, "h2")
    pm = [r.mlp_partial() for r in ranks]
    for r in ranks:
        r.mlp_reduce(pm)
    for r in ranks:
        r.mlp_bwd_slice(r._rows(dout))
    gather(ranks, "d_mlp")
    pb = [r.mlp_bwd_core() for r in ranks]
    for r in ranks:
        r.mlp_bwd_reduce(pb, r._rows(dout))
    gather(ranks, "d_attn")
    pq = [r.attn_bwd_partial() for r in ranks]
    for r in ranks:
        r.attn_bwd_reduce(pq, r._rows(x))
    return {"attn": pa, "mlp": pm, "mlp_bwd": pb, "attn_bwd": pq}


def make_sp_ranks(shards, shared, B, L, heads_per_rank, d, **kw):
    n = len(shards)
    return [SPRankLayer(sh, shared, B, L, heads_per_rank, d, i, n, **kw) for i, sh in enumerate(shards)]


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

    def logits_triples(self, hidden, labels):
        # The logits GEMM and the shard's statistics in one pass (no logits
        # stored): for a forward that needs the loss but not dZ.
        mp.mp_vocab_parallel_logits_xent(hidden, self.E, labels, self.v0, self.tr)
        return self.tr

    def combine(self, triples):
        mp.mp_vocab_xent_combine(triples, self.loss, self.stats, self.mean)
        return self.loss

    def xent_bwd(self, labels, g):
        mp.mp_vocab_parallel_xent_bwd(self.z, labels, self.v0, self.stats, g, self.z)
        return self.z
