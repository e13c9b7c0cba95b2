"""GPU parity: head-partitioned attention (fused QKV GEMM + causal attention)
and its backward against the oracle.  Sequence lengths are ragged against
the 64-key and 64/128-query blocks; the full-size cases use the GPT-2-medium
layer (16 heads of 64) and one rank's 3 heads of 128 of the 8.3B layer."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import TOL, cu, f64, randn, rel_frobenius, say, sync
from megatron_tensor_transformer_02_amd import mp

pytestmark = pytest.mark.gpu


def run_fwd(B, L, K, h, d, causal, seed):
    x = randn(seed, (B * L, K), "bf16")
    w = randn(seed + 1, (3 * h * d, K), "bf16", 0.05 if K <= 256 else 0.02)
    bq = randn(seed + 2, (3 * h * d,), "bf16", 0.1)
    xd, wd, bd = cu(x), cu(w), cu(bq)
    ctx = torch.empty((B * L, h * d), dtype=torch.bfloat16, device="cuda")
    qkv = torch.empty((B * L, 3 * h * d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, h, L), dtype=torch.float32, device="cuda")
    mp.mp_head_attention(xd, wd, bd, B, L, h, d, ctx, qkv, lse, causal)
    sync()
    return x, w, bq, xd, wd, ctx, qkv, lse


def check_core_grads(ws, qkv, dctx, B, L, h, d, causal, seqs=None):
    """dQ, dK and dV (left in the workspace's first T*3hd bf16) against the
    oracle's attention-core backward on the GPU's own projection, each on its
    own so an error in one is not diluted by the others."""
    T, hd = B * L, h * d
    dqkv = f64(ws[:T * 3 * hd * 2].view(torch.bfloat16).reshape(T, 3 * hd))
    q, k, v = O.split_qkv_heads(f64(qkv), B, L, h, d)
    do = f64(dctx).reshape(B, L, h, d).transpose(0, 2, 1, 3)
    sel = list(range(B)) if seqs is None else seqs
    want = O.attention_core_bwd(q[sel], k[sel], v[sel], do[sel], causal)
    got = dqkv.reshape(B, L, 3, h, d)[sel]
    for i, name in enumerate("qkv"):
        err = rel_frobenius(got[:, :, i].transpose(0, 2, 1, 3), want[i])
        assert err <= TOL["bf16"], (name, err)


@pytest.mark.parametrize("B,L,K,h,d,causal", [
    (2, 100, 64, 2, 64, True), (1, 257, 128, 3, 128, True), (2, 70, 96, 1, 64, False),
    (3, 1, 64, 2, 128, True), (1, 200, 256, 2, 128, False),
    # stored-dS backward edges: one whole 64 x 64 tile, one key past a tile,
    # exactly two tiles
    (1, 64, 64, 1, 64, True), (2, 65, 64, 1, 128, False), (1, 128, 64, 2, 128, True),
    # past 4096 keys the few-pairs backward recomputes dS instead of storing it
    (1, 4104, 64, 1, 64, True),
    # either side of the block-count threshold (B h ceil(L/128) = 510 and 512)
    # between 4-wave blocks with the stored dS^T and 8-wave blocks
    (1, 130, 64, 255, 64, True), (1, 130, 64, 256, 64, True)])
def test_head_attention_fwd_bwd(B, L, K, h, d, causal):
    say("attention", B, L, K, h, d, causal)
    x, w, bq, xd, wd, ctx, qkv, lse = run_fwd(B, L, K, h, d, causal, 10)
    wctx, wlse, wqkv = O.head_attention(f64(x), f64(w), f64(bq), B, L, h, d, causal)
    assert rel_frobenius(f64(qkv), wqkv) <= TOL["bf16"]
    # The attention core on the GPU's own projection isolates it from the GEMM.
    q, k, v = O.split_qkv_heads(f64(qkv), B, L, h, d)
    core, core_lse = O.attention_core(q, k, v, causal)
    assert rel_frobenius(f64(ctx), core.transpose(0, 2, 1, 3).reshape(B * L, h * d)) <= TOL["bf16"]
    assert np.max(np.abs(f64(lse) - core_lse)) <= 1e-3
    assert rel_frobenius(f64(ctx), wctx) <= TOL["bf16"]
    dctx = randn(20, (B * L, h * d), "bf16")
    dx = torch.empty((B * L, K), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((3 * h * d, K), dtype=torch.float32, device="cuda")
    db = torch.empty(3 * h * d, dtype=torch.float32, device="cuda")
    ws = torch.empty(mp.lib().mp_head_attention_bwd_workspace(mp.MP_BF16, B, L, K, h, d), dtype=torch.uint8, device="cuda")
    mp.mp_head_attention_bwd(xd, wd, qkv, ctx, lse, cu(dctx), B, L, h, d, dx, dw, db, causal, ws=ws)
    sync()
    check_core_grads(ws, qkv, dctx, B, L, h, d, causal)
    wdx, wdw, wdb = O.head_attention_bwd(f64(x), f64(w), f64(qkv), f64(dctx), B, L, h, d, causal)
    assert rel_frobenius(f64(dx), wdx) <= TOL["bf16"]
    assert rel_frobenius(f64(dw), wdw) <= TOL["bf16"]
    assert rel_frobenius(f64(db), wdb) <= TOL["bf16"]


@pytest.mark.slow
@pytest.mark.parametrize("B,L,K,h,d", [(8, 1024, 1024, 16, 64), (8, 1024, 3072, 3, 128)])
def test_head_attention_full_size(B, L, K, h, d):
    say("attention full", B, L, K, h, d)
    x, w, bq, xd, wd, ctx, qkv, lse = run_fwd(B, L, K, h, d, True, 30)
    q, k, v = O.split_qkv_heads(f64(qkv), B, L, h, d)
    sel = [0, B - 1]  # two whole sequences through the oracle
    core, core_lse = O.attention_core(q[sel], k[sel], v[sel], True)
    got = f64(ctx).reshape(B, L, h, d)[sel].transpose(0, 2, 1, 3)
    assert rel_frobenius(got, core) <= TOL["bf16"]
    assert np.max(np.abs(f64(lse)[sel] - core_lse)) <= 1e-3
    rows = np.random.default_rng(2).choice(B * L, 64, replace=False)
    assert rel_frobenius(f64(qkv)[rows], f64(x)[rows] @ f64(w).T + f64(bq)) <= TOL["bf16"]
    dctx = randn(40, (B * L, h * d), "bf16")
    dx = torch.empty((B * L, K), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((3 * h * d, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(mp.lib().mp_head_attention_bwd_workspace(mp.MP_BF16, B, L, K, h, d), dtype=torch.uint8, device="cuda")
    mp.mp_head_attention_bwd(xd, wd, qkv, ctx, lse, cu(dctx), B, L, h, d, dx, dw, None, True, ws=ws)
    sync()
    check_core_grads(ws, qkv, dctx, B, L, h, d, True, seqs=sel)
    wdx, wdw, _ = O.head_attention_bwd(f64(x), f64(w), f64(qkv), f64(dctx), B, L, h, d, True)
    assert rel_frobenius(f64(dx), wdx) <= TOL["bf16"]
    assert rel_frobenius(f64(dw), wdw) <= TOL["bf16"]
