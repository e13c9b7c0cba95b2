"""GPU parity: LayerNorm forward/backward against the oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import TOL, cu, f64, randn, rel_frobenius, say, sync, tdtype
from megatron_tensor_transformer_02_amd import mp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,T,K", [("bf16", 8192, 1024), ("bf16", 1000, 3072), ("f32", 33, 64),
                                       ("bf16", 5, 8), ("f32", 7, 4092)])
def test_layernorm_fwd_bwd(dtype, T, K):
    say("layernorm", dtype, T, K)
    x = randn(1, (T, K), dtype) * 2 + 0.5
    x = x.to(tdtype(dtype))
    g = (1 + randn(2, (K,), "f32", 0.1)).to(tdtype(dtype))
    b = randn(3, (K,), dtype, 0.1)
    dy = randn(4, (T, K), dtype)
    dres = randn(5, (T, K), dtype)
    y = torch.empty((T, K), dtype=tdtype(dtype), device="cuda")
    mean = torch.empty(T, dtype=torch.float32, device="cuda")
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    xd = cu(x)
    mp.mp_layernorm(xd, cu(g), cu(b), y, mean, rstd, 1e-5)
    sync()
    wy, wm, wr = O.layernorm(f64(x), f64(g), f64(b), 1e-5)
    assert rel_frobenius(f64(y), wy) <= TOL[dtype]
    assert rel_frobenius(f64(mean), wm) <= 1e-5
    assert rel_frobenius(f64(rstd), wr) <= 1e-5
    dx = torch.empty_like(y)
    dg = torch.empty(K, dtype=torch.float32, device="cuda")
    db = torch.empty(K, dtype=torch.float32, device="cuda")
    mp.mp_layernorm_bwd(xd, cu(g), mean, rstd, cu(dy), dx, cu(dres), dg, db)
    sync()
    wdx, wdg, wdb = O.layernorm_bwd(f64(dy), f64(x), f64(g), wm, wr)
    assert rel_frobenius(f64(dx), wdx + f64(dres)) <= TOL[dtype]
    # dgamma and dbeta are fp32 sums over T rows of terms of either sign:
    # fp32 summation error scales with the sum of the terms' magnitudes, not
    # with the (cancelling) sum, so each column is held to 1e-5 of that.
    xhat = (f64(x) - wm[:, None]) * wr[:, None]
    assert np.all(np.abs(f64(dg) - wdg) <= 1e-5 * np.abs(f64(dy) * xhat).sum(axis=0))
    assert np.all(np.abs(f64(db) - wdb) <= 1e-5 * np.abs(f64(dy)).sum(axis=0))
    assert rel_frobenius(f64(db), wdb) <= 1e-5
    assert rel_frobenius(f64(dg), wdg) <= TOL[dtype]
