"""The no-allocation entry point mp_row_linear_partial_bwd_static against
mp_row_linear_partial_bwd, through the C ABI: two calls in a row on the
library's static scratch (the second with a smaller input, so it runs over
what the first left there) give the workspace call's results bit for bit,
match the oracle, and allocate no device memory.  Also the host-side
rejections, which need no GPU."""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import TOL, cu, f64, randn, rel_frobenius, say, sync
from megatron_tensor_transformer_02_amd import mp

ALIGNED = 0x10000


def test_static_variant_rejects_before_any_work():
    lib = mp.lib()
    cap = lib.mp_row_linear_partial_bwd_static_max_bytes()
    assert cap == 64 << 20
    # 32768 tokens into a [3072, 3072] weight: split-K partials beyond the cap.
    assert lib.mp_row_linear_partial_bwd_workspace(mp.MP_BF16, 32768, 3072, 3072) > cap
    rc = lib.mp_row_linear_partial_bwd_static(mp.MP_BF16, 32768, 3072, 3072, ALIGNED, ALIGNED, ALIGNED, ALIGNED,
                                              ALIGNED, None)
    assert rc == -6 and "static" in lib.mp_last_error().decode()
    rc = lib.mp_row_linear_partial_bwd_static(mp.MP_BF16, 8192, 384, 3072, ALIGNED, None, ALIGNED, ALIGNED,
                                              ALIGNED, None)
    assert rc == -1
    rc = lib.mp_row_linear_partial_bwd_static(mp.MP_BF16, 8192, 384, 3072, ALIGNED, ALIGNED, ALIGNED + 8, ALIGNED,
                                              ALIGNED, None)
    assert rc == -5
    rc = lib.mp_row_linear_partial_bwd_static(mp.MP_BF16, 8192, 384, 3076, ALIGNED, ALIGNED, ALIGNED, ALIGNED,
                                              ALIGNED, None)
    assert rc == -2


@pytest.mark.gpu
def test_static_scratch_matches_workspace_call_twice():
    lib = mp.lib()
    cases = [(8192, 1536, 3072), (2048, 384, 3072), (1000, 200, 264)]  # each call smaller than the last
    for i, (T, Fi, K) in enumerate(cases):
        say("no-alloc row bwd", T, Fi, K)
        need = lib.mp_row_linear_partial_bwd_workspace(mp.MP_BF16, T, Fi, K)
        assert 0 < need <= lib.mp_row_linear_partial_bwd_static_max_bytes()  # split-K: the scratch is used
        y, b, dout = randn(50 + i, (T, Fi), "bf16"), randn(60 + i, (K, Fi), "bf16", 0.02), randn(70 + i, (T, K), "bf16")
        yd, bd, dd = cu(y), cu(b), cu(dout)
        dy_ref = torch.empty((T, Fi), dtype=torch.bfloat16, device="cuda")
        db_ref = torch.empty((K, Fi), dtype=torch.float32, device="cuda")
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        mp.mp_row_linear_partial_bwd(yd, bd, dd, dy_ref, db_ref, ws=ws)
        dy = torch.full((T, Fi), 7.0, dtype=torch.bfloat16, device="cuda")
        db = torch.full((K, Fi), 7.0, dtype=torch.float32, device="cuda")
        sync()
        before = torch.cuda.memory_allocated()
        stream = torch.cuda.current_stream().cuda_stream
        rc = lib.mp_row_linear_partial_bwd_static(mp.MP_BF16, T, Fi, K, ctypes.c_void_p(yd.data_ptr()),
                                                  ctypes.c_void_p(bd.data_ptr()), ctypes.c_void_p(dd.data_ptr()),
                                                  ctypes.c_void_p(dy.data_ptr()), ctypes.c_void_p(db.data_ptr()),
                                                  ctypes.c_void_p(stream))
        assert rc == 0, lib.mp_last_error().decode()
        sync()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(dy, dy_ref) and torch.equal(db, db_ref)
        rows = np.random.default_rng(i).choice(T, min(T, 256), replace=False)
        wdy = f64(dout)[rows] @ f64(b)
        assert rel_frobenius(f64(dy)[rows], wdy) <= TOL["bf16"]
        assert rel_frobenius(f64(db), f64(dout).T @ f64(y)) <= TOL["bf16"]
