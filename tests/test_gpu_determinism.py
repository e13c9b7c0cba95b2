"""Run-to-run determinism of every entry point: each call runs twice on the
same inputs (with other work in between) and every output must be identical
byte for byte.  All reductions in the library use a fixed order -- split-K
partials summed in split order, column sums over fixed slabs, the shard
reduce in shard order, LayerNorm statistics as fixed-order block sums, the
MoE permutation by scan instead of atomics -- so a difference means a race or
an order that depends on scheduling.  Shapes span several tiles with ragged
tails."""

import numpy as np
import pytest
import torch

from gpu_util import cu, mask_bits, randn, say, sync
from megatron_tensor_transformer_02_amd import mp

pytestmark = pytest.mark.gpu

bf, f32 = torch.bfloat16, torch.float32


def E(*shape, dtype=bf):
    # zero-filled, so entries a call leaves untouched (permutation slots past
    # the routed rows) compare equal too
    return torch.zeros(shape, dtype=dtype, device="cuda")


def case_column_fwd_bwd():
    T, K, F = 700, 520, 392
    x, a, ab, dy = cu(randn(1, (T, K), "bf16")), cu(randn(2, (F, K), "bf16", .05)), cu(randn(3, (F,), "bf16", .1)), \
        cu(randn(4, (T, F), "bf16"))
    y, z, dx, da, dab = E(T, F), E(T, F), E(T, K), E(F, K, dtype=f32), E(F, dtype=f32)
    mp.mp_column_linear_gelu(x, a, ab, "erf", y, z)
    mp.mp_column_linear_gelu_bwd(x, a, z, dy, "erf", dx, da, dab)
    return [y, z, dx, da, dab]


def case_row_fwd_bwd():
    T, F, K = 2048, 384, 1000
    y, b, do, z = cu(randn(5, (T, F), "bf16")), cu(randn(6, (K, F), "bf16", .05)), cu(randn(7, (T, K), "bf16")), \
        cu(randn(8, (T, F), "bf16"))
    p, dy, db, dz, db2 = E(T, K), E(T, F), E(K, F, dtype=f32), E(T, F), E(K, F, dtype=f32)
    mp.mp_row_linear_partial(y, b, p)
    mp.mp_row_linear_partial_bwd(y, b, do, dy, db)  # split-K weight gradient
    mp.mp_row_linear_partial_bwd_dact(y, b, do, z, "tanh", dz, db2)
    return [p, dy, db, dz, db2]


def case_logits_fp32():
    T, K, V = 513, 264, 1096
    h, e = cu(randn(9, (T, K), "bf16")), cu(randn(10, (V, K), "bf16", .05))
    zl = E(T, V, dtype=f32)
    mp.mp_column_linear_gelu(h, e, None, "none", zl)
    return [zl]


def case_shard_reduce_dropout():
    n, rows, cols = 8, 300, 1032
    parts = [cu(randn(20 + j, (rows, cols), "bf16")) for j in range(n)]
    bias, res = cu(randn(30, (cols,), "bf16", .1)), cu(randn(31, (rows, cols), "bf16"))
    out, mask = E(rows, cols), mask_bits(rows * cols)
    mp.mp_shard_reduce(parts, out, bias, res, 0.1, 1234, 5, 0, mask)
    x, y = cu(randn(32, (rows * cols,), "bf16")), E(rows * cols)
    mp.mp_shared_seed_dropout(x, y, 0.3, 99, 2, 16)
    dx, dbias = E(rows, cols), E(cols, dtype=f32)
    mp.mp_dropout_mask_bwd(parts[0], mask, 0.1, dx, dbias)
    db = E(cols, dtype=f32)
    mp.mp_bias_grad(parts[1], db)
    gathered = E(4 * 75, cols)
    mp.mp_all_gather_rows([parts[j][:75] for j in range(4)], gathered)
    return [out, mask, y, dx, dbias, db, gathered]


def case_fused_reduce_layernorm():
    n, rows, cols = 8, 257, 3072
    parts = [cu(randn(40 + j, (rows, cols), "bf16")) for j in range(n)]
    bias, res = cu(randn(50, (cols,), "bf16", .1)), cu(randn(51, (rows, cols), "bf16"))
    g, b = cu(randn(52, (cols,), "bf16", .2) + 1), cu(randn(53, (cols,), "bf16", .1))
    out, y, mean, rstd, mask = E(rows, cols), E(rows, cols), E(rows, dtype=f32), E(rows, dtype=f32), \
        mask_bits(rows * cols)
    mp.mp_shard_reduce_layernorm(parts, out, g, b, y, mean, rstd, bias=bias, residual=res, p=0.1, seed=3, offset=1,
                                 mask_out=mask)
    dx, dg, dbeta = E(rows, cols), E(cols, dtype=f32), E(cols, dtype=f32)
    mp.mp_shard_reduce_layernorm_bwd(parts, out, g, mean, rstd, dx, res, dg, dbeta)
    dx2, dg2, db2, ddrop, dbias = E(rows, cols), E(cols, dtype=f32), E(cols, dtype=f32), E(rows, cols), \
        E(cols, dtype=f32)
    mp.mp_shard_reduce_layernorm_bwd_dropout(parts, out, g, mean, rstd, dx2, 0.1, mask, ddrop, dres=res, dgamma=dg2,
                                             dbeta=db2, dbias=dbias)
    return [out, y, mean, rstd, mask, dx, dg, dbeta, dx2, dg2, db2, ddrop, dbias]


def case_layernorm():
    T, K = 1000, 3072
    x, g, b, dy = cu(randn(60, (T, K), "bf16")), cu(randn(61, (K,), "bf16", .2) + 1), cu(randn(62, (K,), "bf16", .1)), \
        cu(randn(63, (T, K), "bf16"))
    y, mean, rstd = E(T, K), E(T, dtype=f32), E(T, dtype=f32)
    mp.mp_layernorm(x, g, b, y, mean, rstd)
    dx, dg, db = E(T, K), E(K, dtype=f32), E(K, dtype=f32)
    mp.mp_layernorm_bwd(x, g, mean, rstd, dy, dx, None, dg, db)
    return [y, mean, rstd, dx, dg, db]


def case_attention(d=128, h=3):
    B, L, K = 2, 700, 384
    x, w, bq = cu(randn(70, (B * L, K), "bf16")), cu(randn(71, (3 * h * d, K), "bf16", .05)), \
        cu(randn(72, (3 * h * d,), "bf16", .1))
    ctx, qkv, lse = E(B * L, h * d), E(B * L, 3 * h * d), E(B, h, L, dtype=f32)
    mp.mp_head_attention(x, w, bq, B, L, h, d, ctx, qkv, lse)
    dctx = cu(randn(73, (B * L, h * d), "bf16"))
    dx, dw, db = E(B * L, K), E(3 * h * d, K, dtype=f32), E(3 * h * d, dtype=f32)
    ws = torch.empty(mp.lib().mp_head_attention_bwd_workspace(mp.MP_BF16, B, L, K, h, d), dtype=torch.uint8,
                     device="cuda")
    mp.mp_head_attention_bwd(x, w, qkv, ctx, lse, dctx, B, L, h, d, dx, dw, db, ws=ws)
    return [ctx, qkv, lse, dx, dw, db, ws[:B * L * 3 * h * d * 2]]


def case_attention_d64():
    return case_attention(64, 4)


def case_vocab():
    T, V, K, n = 1000, 1024, 264, 2
    vi = V // n
    ids = torch.from_numpy(np.random.default_rng(80).integers(0, V, T).astype(np.int32)).cuda()
    emb, dout = cu(randn(81, (V, K), "bf16", .05)), cu(randn(82, (T, K), "bf16"))
    part, de = E(T, K), E(vi, K, dtype=f32)
    mp.mp_vocab_parallel_embedding(ids, emb[:vi], 0, part)
    mp.mp_vocab_parallel_embedding_bwd(ids, dout, 0, de)
    z = [cu(randn(83 + j, (T, vi), "f32") * 3) for j in range(n)]
    tr = [E(T, 3, dtype=f32) for _ in range(n)]
    for j in range(n):
        mp.mp_vocab_parallel_xent(z[j], ids, j * vi, tr[j])
    loss, stats, mean = E(T, dtype=f32), E(T, 2, dtype=f32), E(1, dtype=f32)
    mp.mp_vocab_xent_combine(tr, loss, stats, mean)
    dz = E(T, vi, dtype=f32)
    mp.mp_vocab_parallel_xent_bwd(z[0], ids, 0, stats, 1.0 / T, dz)
    h = cu(randn(90, (T, K), "bf16"))
    trf = E(T, 3, dtype=f32)
    mp.mp_vocab_parallel_logits_xent(h, emb[:vi], ids, 0, trf)
    return [part, de, *tr, loss, stats, mean, dz, trf]


def _moe_inputs(T=300, Hd=256, Fe=136, experts=32, e_local=8, topk=8, seed=5):
    rng = np.random.default_rng(seed)
    ids = torch.from_numpy(np.stack([rng.permutation(experts)[:topk] for _ in range(T)]).astype(np.int32)).cuda()
    w = rng.random((T, topk)).astype(np.float32)
    w = torch.from_numpy(w / w.sum(axis=1, keepdims=True)).cuda()
    x = torch.from_numpy(rng.standard_normal((T, Hd), dtype=np.float32)).to(bf).cuda()
    wgu = torch.from_numpy(rng.standard_normal((e_local, 2 * Fe, Hd), dtype=np.float32) * .1).to(bf).cuda()
    wd = torch.from_numpy(rng.standard_normal((e_local, Hd, Fe), dtype=np.float32) * .1).to(bf).cuda()
    dout = torch.from_numpy(rng.standard_normal((T, Hd), dtype=np.float32)).to(bf).cuda()
    return ids, w, x, wgu, wd, dout


def case_moe(shape=None):
    ids, w, x, wgu, wd, dout = _moe_inputs(**(shape or {}))
    T, Hd = x.shape
    topk = ids.shape[1]
    e_local, two_fe, _ = wgu.shape
    res = []
    for fwd in (mp.mp_grouped_expert_gemm, mp.mp_grouped_expert_gemm_weighted_act):
        out, perm, offs = E(T, Hd), E(T * topk, dtype=torch.int32), E(e_local + 1, dtype=torch.int32)
        fwd(x, ids, w, wgu, wd, 0, out, perm, offs)
        res += [out, perm, offs]
    for wa in (False, True):
        out, gu = E(T, Hd), E(T * topk, two_fe)
        fws = mp.mp_grouped_expert_gemm_fwd_train(x, ids, w, wgu, wd, 0, out, gu, weighted_act=wa)
        dx, dwgu, dwd, dtw = E(T, Hd), E(e_local, two_fe, Hd, dtype=f32), E(e_local, Hd, two_fe // 2, dtype=f32), \
            E(T, topk, dtype=f32)
        mp.mp_grouped_expert_gemm_bwd(x, w, wgu, wd, dout, gu, fws, dx, dwgu, dwd, dtw, weighted_act=wa)
        res += [out, gu, dx, dwgu, dwd, dtw]
    return res


def case_moe_split_sparse():
    # Sparse experts whose launches split the k-range (fp32 partials + reduce).
    return case_moe(dict(T=300, Hd=1096, Fe=1032, experts=32, e_local=8, topk=2))


def case_moe_mxfp8():
    ids, w, x, wgu, wd, _ = _moe_inputs(T=200, Hd=256, Fe=128, experts=16, e_local=4, topk=4)
    T, Hd = x.shape
    topk = ids.shape[1]
    e_local, two_fe, _ = wgu.shape
    fe = two_fe // 2
    qg, sg = E(e_local, two_fe, Hd, dtype=torch.uint8), E(e_local, two_fe, mp.mxfp8_scale_width(Hd), dtype=torch.uint8)
    qd, sd = E(e_local, Hd, fe, dtype=torch.uint8), E(e_local, Hd, mp.mxfp8_scale_width(fe), dtype=torch.uint8)
    for e in range(e_local):
        mp.mp_mxfp8_quantize(wgu[e], qg[e], sg[e])
        mp.mp_mxfp8_quantize(wd[e], qd[e], sd[e])
    out, perm, offs = E(T, Hd), E(T * topk, dtype=torch.int32), E(e_local + 1, dtype=torch.int32)
    mp.mp_grouped_expert_gemm_mxfp8(x, ids, w, qg, sg, qd, sd, 0, out, perm, offs)
    return [qg, sg, qd, sd, out, perm, offs]


CASES = {name[5:]: fn for name, fn in globals().items() if name.startswith("case_")}


@pytest.mark.parametrize("name", sorted(CASES))
def test_two_runs_are_bit_identical(name):
    say("determinism", name)
    first = [t.clone() for t in CASES[name]()]
    junk = torch.randn(1 << 22, device="cuda")  # other work (and allocator churn) in between
    junk.mul_(2).add_(1)
    del junk
    mp._ws_cache.clear()
    second = CASES[name]()
    sync()
    assert len(first) == len(second)
    for i, (a, b) in enumerate(zip(first, second)):
        assert a.shape == b.shape and a.dtype == b.dtype, (name, i)
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b), (name, i)
