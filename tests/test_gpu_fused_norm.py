"""GPU parity: the shard reduce fused with the LayerNorm it feeds, forward
and backward, against the oracle (reduce, dropout, LayerNorm and its
backward composed) and against the unfused GPU calls.  The reduced sum and
the dropout mask are bit-identical to the unfused path; the LayerNorm
statistics are block sums in another fixed order, so the normalised outputs
and gradients agree to rounding.  Repeated calls are bit-identical."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import TOL, cu, f64, mask_bits, randn, rel_frobenius, say, sync, tdtype, unpack_bits
from megatron_tensor_transformer_02_amd import mp

pytestmark = pytest.mark.gpu

CASES = [
    ("f32", 2, 32, 64, 0.1),        # tiny workload: N=2 fp32
    ("bf16", 8, 77, 3072, 0.1),     # 8-way, the 8.3B-config hidden size, ragged rows
    ("bf16", 3, 130, 136, 0.0),     # odd N, partial last vector group, no dropout
    ("bf16", 1, 5, 8, 0.5),         # N=1, one vector per row
    ("bf16", 16, 33, 1024, 0.9),    # maximum N, heavy dropout
    ("bf16", 8, 2048, 3072, 0.1),   # a quarter of the full token count
    # rows wider than 4096 values: 16-wave blocks, no next-row prefetch
    ("bf16", 8, 40, 7168, 0.1), ("f32", 3, 24, 4096, 0.0), ("bf16", 12, 20, 8192, 0.1),
]


@pytest.mark.parametrize("dtype,n,rows,cols,p", CASES)
def test_reduce_layernorm_fwd(dtype, n, rows, cols, p):
    say("reduce+LN fwd", dtype, n, rows, cols, p)
    parts = [cu(randn(20 + j, (rows, cols), dtype)) for j in range(n)]
    bias, res = cu(randn(60, (cols,), dtype, 0.1)), cu(randn(61, (rows, cols), dtype))
    gamma, beta = cu(randn(62, (cols,), dtype, 0.2) + 1), cu(randn(63, (cols,), dtype, 0.1))
    seed, off, ib = 0x0BADC0FFEE, 3, 8
    t = tdtype(dtype)
    out, y = torch.empty((rows, cols), dtype=t, device="cuda"), torch.empty((rows, cols), dtype=t, device="cuda")
    mean, rstd = torch.empty(rows, device="cuda"), torch.empty(rows, device="cuda")
    mask = mask_bits(rows * cols)
    mp.mp_shard_reduce_layernorm(parts, out, gamma, beta, y, mean, rstd, bias=bias, residual=res, p=p, seed=seed,
                                 offset=off, index_base=ib, mask_out=mask)
    # unfused GPU path
    out2, y2 = torch.empty_like(out), torch.empty_like(y)
    mean2, rstd2 = torch.empty_like(mean), torch.empty_like(rstd)
    mask2 = torch.empty_like(mask)
    mp.mp_shard_reduce(parts, out2, bias, res, p, seed, off, ib, mask2)
    mp.mp_layernorm(out2, gamma, beta, y2, mean2, rstd2)
    sync()
    assert torch.equal(out, out2) and torch.equal(mask, mask2)
    assert rel_frobenius(f64(y), f64(y2)) <= TOL[dtype]
    assert rel_frobenius(f64(mean), f64(mean2)) <= 1e-5 and rel_frobenius(f64(rstd), f64(rstd2)) <= 1e-5
    # oracle: the reduce from the inputs, LayerNorm of the stored (rounded) sum
    acc = sum(f64(t_) for t_ in parts) + f64(bias)
    want_pre, keep = O.dropout(acc, p, seed, off, start=ib)
    assert np.array_equal(unpack_bits(mask, rows * cols).reshape(rows, cols), keep)
    assert rel_frobenius(f64(out), want_pre + f64(res)) <= TOL[dtype]
    wy, wm, wr = O.layernorm(f64(out), f64(gamma), f64(beta))
    assert rel_frobenius(f64(y), wy) <= TOL[dtype]
    # A row mean of values of either sign cancels: fp32 summation error is
    # bounded relative to the mean magnitude of the row's values.
    assert np.all(np.abs(f64(mean) - wm) <= 1e-5 * np.abs(f64(out)).mean(axis=1))
    assert rel_frobenius(f64(rstd), wr) <= 1e-5


@pytest.mark.parametrize("dtype,n,rows,cols,p", CASES)
def test_reduce_layernorm_bwd(dtype, n, rows, cols, p):
    say("reduce+LN bwd", dtype, n, rows, cols)
    parts = [cu(randn(30 + j, (rows, cols), dtype)) for j in range(n)]
    x = cu(randn(70, (rows, cols), dtype))
    gamma, beta = cu(randn(71, (cols,), dtype, 0.2) + 1), cu(randn(72, (cols,), dtype, 0.1))
    dres = cu(randn(73, (rows, cols), dtype))
    t = tdtype(dtype)
    y = torch.empty((rows, cols), dtype=t, device="cuda")
    mean, rstd = torch.empty(rows, device="cuda"), torch.empty(rows, device="cuda")
    mp.mp_layernorm(x, gamma, beta, y, mean, rstd)
    dx = torch.empty((rows, cols), dtype=t, device="cuda")
    dg, db = torch.empty(cols, device="cuda"), torch.empty(cols, device="cuda")
    mp.mp_shard_reduce_layernorm_bwd(parts, x, gamma, mean, rstd, dx, dres, dg, db)
    # unfused GPU path
    dy = torch.empty((rows, cols), dtype=t, device="cuda")
    mp.mp_shard_reduce(parts, dy)
    dx2 = torch.empty_like(dx)
    mp.mp_layernorm_bwd(x, gamma, mean, rstd, dy, dx2, dres)
    sync()
    assert rel_frobenius(f64(dx), f64(dx2)) <= TOL[dtype]
    # oracle: LayerNorm backward of the (rounded) reduced gradient
    wdx, wdg, wdb = O.layernorm_bwd(f64(dy), f64(x), f64(gamma), f64(mean), f64(rstd))
    assert rel_frobenius(f64(dx), wdx + f64(dres)) <= TOL[dtype]
    assert rel_frobenius(f64(dg), wdg) <= 1e-5
    assert rel_frobenius(f64(db), wdb) <= 1e-5
    # deterministic: a second call gives the same bits
    dg2, db2 = torch.empty_like(dg), torch.empty_like(db)
    mp.mp_shard_reduce_layernorm_bwd(parts, x, gamma, mean, rstd, dx2, dres, dg2, db2)
    sync()
    assert torch.equal(dg, dg2) and torch.equal(db, db2) and torch.equal(dx, dx2)
    # and a repeated forward, too
    y3 = torch.empty_like(x)
    mp.mp_shard_reduce_layernorm(parts, dx2, gamma, beta, y3)
    mp.mp_shard_reduce_layernorm(parts, dx, gamma, beta, y)
    sync()
    assert torch.equal(y, y3)


def test_reduce_layernorm_bwd_aliasing_and_no_params():
    # dres aliasing dx (the layer's usage pattern allows it) and no parameter gradients.
    say("reduce+LN bwd alias")
    rows, cols, n = 64, 256, 4
    parts = [cu(randn(40 + j, (rows, cols), "bf16")) for j in range(n)]
    x = cu(randn(80, (rows, cols), "bf16"))
    gamma, beta = cu(randn(81, (cols,), "bf16", 0.2) + 1), cu(randn(82, (cols,), "bf16", 0.1))
    y = torch.empty_like(x)
    mean, rstd = torch.empty(rows, device="cuda"), torch.empty(rows, device="cuda")
    mp.mp_layernorm(x, gamma, beta, y, mean, rstd)
    d = cu(randn(83, (rows, cols), "bf16"))
    ref = d.clone()
    mp.mp_shard_reduce_layernorm_bwd(parts, x, gamma, mean, rstd, d, d)
    dy = torch.empty_like(x)
    mp.mp_shard_reduce(parts, dy)
    want = torch.empty_like(x)
    mp.mp_layernorm_bwd(x, gamma, mean, rstd, dy, want, ref)
    sync()
    assert rel_frobenius(f64(d), f64(want)) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,n,rows,cols,p", CASES)
def test_reduce_layernorm_bwd_dropout(dtype, n, rows, cols, p):
    """The fused backward that also applies the next branch's dropout (from
    the keep bits its forward saved) to dx and sums its columns: dx and the
    parameter gradients are those of the plain fused backward bit for bit,
    ddrop is a separate dropout-backward pass over dx bit for bit, dbias
    matches that pass's column sums and the oracle."""
    say("reduce+LN bwd + dropout", dtype, n, rows, cols, p)
    parts = [cu(randn(90 + j, (rows, cols), dtype)) for j in range(n)]
    x = cu(randn(74, (rows, cols), dtype))
    gamma, beta = cu(randn(75, (cols,), dtype, 0.2) + 1), cu(randn(76, (cols,), dtype, 0.1))
    dres = cu(randn(77, (rows, cols), dtype))
    t = tdtype(dtype)
    y = torch.empty((rows, cols), dtype=t, device="cuda")
    mean, rstd = torch.empty(rows, device="cuda"), torch.empty(rows, device="cuda")
    mp.mp_layernorm(x, gamma, beta, y, mean, rstd)
    seed, off = 0xFEEDFACE12, 5
    bits = mask_bits(rows * cols)  # the branch's forward dropout, saved as bits
    mp.mp_shared_seed_dropout(x, torch.empty_like(x), p, seed, off, 0, bits)
    dx, dd = torch.empty((rows, cols), dtype=t, device="cuda"), torch.empty((rows, cols), dtype=t, device="cuda")
    dg, db, dbias = (torch.empty(cols, device="cuda") for _ in range(3))
    mp.mp_shard_reduce_layernorm_bwd_dropout(parts, x, gamma, mean, rstd, dx, p, bits, dd, dres=dres, dgamma=dg,
                                             dbeta=db, dbias=dbias)
    # unfused GPU path: plain fused backward, then dropout backward + bias gradient
    dx2 = torch.empty_like(dx)
    dg2, db2, dbias2 = (torch.empty(cols, device="cuda") for _ in range(3))
    mp.mp_shard_reduce_layernorm_bwd(parts, x, gamma, mean, rstd, dx2, dres, dg2, db2)
    dd2 = torch.empty_like(dd)
    mp.mp_shared_seed_dropout(dx2, dd2, p, seed, off, 0)
    mp.mp_bias_grad(dd2, dbias2)
    sync()
    assert torch.equal(dx, dx2) and torch.equal(dg, dg2) and torch.equal(db, db2)
    assert torch.equal(dd, dd2)
    assert rel_frobenius(f64(dbias), f64(dbias2)) <= 1e-5
    # oracle: dropout of the stored dx (mask from the shared-seed generator) and its column sums
    want_dd, _ = O.dropout(f64(dx), p, seed, off)
    assert rel_frobenius(f64(dd), want_dd) <= TOL[dtype]
    assert rel_frobenius(f64(dbias), O.bias_grad(f64(dd))) <= 1e-5
    # without dbias (no workspace needed for it) the outputs are unchanged
    dd3 = torch.empty_like(dd)
    mp.mp_shard_reduce_layernorm_bwd_dropout(parts, x, gamma, mean, rstd, dx2, p, bits, dd3, dres=dres)
    sync()
    assert torch.equal(dd3, dd) and torch.equal(dx2, dx)
