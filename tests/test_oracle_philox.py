"""Pins for the oracle's shared-seed dropout (CPU only).

The pages fix only that every device applies the same dropout mask
(MLM-review, "key terms").  The generator is Philox4x32-10 from its published
definition; its stream is pinned here against PyTorch's own, independently
written Philox4x32-10 engine (ATen ``PhiloxRNGEngine.h``), compiled from the
installed header.  Conformance to the paper's known-answer vectors is "parity
unpinned": those vectors are not available here.
"""

import ctypes
import math
import os
import subprocess
import tempfile
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle.philox import (_W0, _W1, dropout, dropout_keep_mask, dropout_threshold,
                           philox4x32_10)

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def torch_philox():
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    tmp = tempfile.mkdtemp(prefix="torch_philox_")
    so = os.path.join(tmp, "tp.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-I" + inc,
                    os.path.join(HERE, "_torch_philox.cpp"), "-o", so], check=True)
    lib = ctypes.CDLL(so)
    lib.torch_philox4.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                  ctypes.POINTER(ctypes.c_uint32)]

    def call(seed, subsequence, offset):
        out = (ctypes.c_uint32 * 4)()
        lib.torch_philox4(seed, subsequence, offset, out)
        return [int(v) for v in out]
    return call


def test_weyl_constants_closed_form():
    # W0 = floor(2^32 * (golden ratio - 1)), W1 = floor(2^32 * (sqrt(3) - 1)).
    getcontext().prec = 50
    phi_frac = (Decimal(5).sqrt() - 1) / 2
    assert int(_W0) == int(phi_frac * (1 << 32))
    assert int(_W1) == int((Decimal(3).sqrt() - 1) * (1 << 32))


@pytest.mark.parametrize("seed,subseq,blk", [
    (0, 0, 0), (1, 0, 0), (0, 1, 0), (0, 0, 1), (123456789, 7, 5),
    (2**64 - 1, 2**40 + 3, 2**33 + 9), (0xDEADBEEFCAFEF00D, 2**32 - 1, 2**32 - 1),
])
def test_block_function_matches_torch(torch_philox, seed, subseq, blk):
    ref = torch_philox(seed, subseq, blk)
    got = philox4x32_10(blk & 0xFFFFFFFF, blk >> 32, subseq & 0xFFFFFFFF, subseq >> 32,
                        seed & 0xFFFFFFFF, seed >> 32)
    assert [int(v) for v in got] == ref


def test_stream_layout_matches_torch(torch_philox):
    # Element j uses word j % 4 of the block at counter (j // 4, offset).
    seed, offset, p = 0x1234_5678_9ABC_DEF0, 77, 0.25
    n = 4 * 40 + 3
    keep = dropout_keep_mask(n, p, seed, offset)
    thr = dropout_threshold(p)
    want = []
    for blk in range((n + 3) // 4):
        want += [w >= thr for w in torch_philox(seed, offset, blk)]
    assert keep.tolist() == want[:n]


def test_threshold_from_float32_p():
    # p crosses the boundary as float32; 0.1f = 0.100000001490116...
    assert dropout_threshold(0.1) == 429496736
    assert dropout_threshold(0.0) == 0
    assert dropout_threshold(0.5) == 2**31
    with pytest.raises(ValueError):
        dropout_threshold(1.0)


def test_p_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((7, 13))
    y, keep = dropout(x, 0.0, 5, 9)
    assert keep.all() and np.array_equal(y, x)


def test_keep_rate_binomial():
    n, p = 200_000, 0.1
    keep = dropout_keep_mask(n, p, 42, 3)
    mean, sd = n * (1 - p), math.sqrt(n * p * (1 - p))
    assert abs(keep.sum() - mean) < 5 * sd


def test_scale_and_start_offset_consistency():
    x = np.random.default_rng(1).standard_normal(1000)
    y, keep = dropout(x, 0.3, 11, 2)
    scale = 1.0 / (1.0 - float(np.float32(0.3)))
    assert np.allclose(y[keep], x[keep] * scale, rtol=0, atol=0)
    assert np.all(y[~keep] == 0)
    # A slice starting at flat index s draws the same words as the whole tensor.
    tail = dropout_keep_mask(600, 0.3, 11, 2, start=400)
    assert np.array_equal(tail, keep[400:])


def test_mask_depends_on_seed_and_offset():
    a = dropout_keep_mask(4096, 0.5, 1, 0)
    assert not np.array_equal(a, dropout_keep_mask(4096, 0.5, 2, 0))
    assert not np.array_equal(a, dropout_keep_mask(4096, 0.5, 1, 1))
    assert np.array_equal(a, dropout_keep_mask(4096, 0.5, 1, 0))
