"""Pins for the oracle's MXFP8 pieces (CPU only).

The E4M3 decode of all 256 codes and the round-to-nearest-even encode against
PyTorch's independent float8_e4m3fn conversion (below 464, where that
conversion does not turn to NaN); saturation above 448; the shared exponent
against its closed form on exact powers of two; exact round trips of values
already on the MX grid; the per-element error bound of the format; and the
MXFP8 expert shard, with the activation's rounding and quantisation off,
against the fp64 shard on the dequantised operands (MOE-core, technical
summary 2.5: expert GEMMs in low precision, router and weights' master copies
high precision).
"""

import numpy as np
import pytest
import torch

import oracle as O

RNG = np.random.default_rng(2024)


def test_e4m3_decode_matches_torch():
    want = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([O.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x08) == 2.0 ** -6 and O.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_round_matches_torch_below_464():
    mags = np.concatenate([
        2.0 ** RNG.uniform(-12, np.log2(463.9), 20000),             # every binade, subnormals included
        np.array([O.e4m3_value(c) for c in range(0x7E)]),            # grid points
        (np.array([O.e4m3_value(c) for c in range(0x7E)]) +
         np.array([O.e4m3_value(c + 1) for c in range(0x7E)])) / 2,  # exact midpoints (ties)
        [0.0, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, 463.0]])
    vals = mags * np.where(RNG.random(mags.size) < 0.5, -1.0, 1.0)
    vals = vals.astype(np.float32).astype(np.float64)  # representable in fp32 for torch
    want = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_round(vals)
    assert np.array_equal(got, want)


def test_e4m3_round_saturates():
    v = np.array([464.0, 479.9, 480.0, 1e4, -500.0, -1e30])
    assert list(O.e4m3_round(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_shared_exponent_closed_form():
    e = np.arange(-126, 128)
    assert np.array_equal(O.shared_exponent(2.0 ** e), np.clip(e - 8, -127, 127))
    assert np.array_equal(O.shared_exponent(2.0 ** e * 1.999), np.clip(e - 8, -127, 127))
    assert O.shared_exponent(0.0) == -127 and O.shared_exponent(2.0 ** -130) == -127


def test_grid_values_round_trip_exactly():
    rows, k = 6, 96
    codes = RNG.integers(0, 0x7F, (rows, k)).astype(np.uint8) | (RNG.integers(0, 2, (rows, k)) << 7).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30  # no NaN codes
    codes[:, ::32] = 0x78  # 256 = 2^8 in every block: its maximum lies in [2^8, 2^9), fixing the exponent
    se = RNG.integers(-20, 20, (rows, k // 32))
    scales = np.full((rows, O.scale_width(k)), 127, dtype=np.uint8)
    scales[:, :k // 32] = se + 127
    x = O.mx_dequantize(codes, scales)
    q, s = O.mx_quantize(x)
    assert np.array_equal(s, scales)
    assert np.array_equal(O.mx_dequantize(q, s), x)
    assert np.array_equal(q[x != 0], codes[x != 0])


def test_quantize_error_bound_and_layout():
    rows, k = 5, 160  # 5 blocks: a ragged last 128-column group in the scale layout
    x = RNG.standard_normal((rows, k)) * 2.0 ** RNG.integers(-30, 30, (rows, 1))
    x[2, 32:64] = 0.0  # an all-zero block
    q, s = O.mx_quantize(x)
    assert s.shape == (rows, 8) and np.all(s[:, 5:] == 127) and s[2, 1] == 0
    d = O.mx_dequantize(q, s)
    scale = np.repeat(2.0 ** (s[:, :5].astype(np.int64) - 127), 32, axis=1)
    normal = np.abs(x) / scale >= 2.0 ** -6
    sat = np.abs(x) / scale > 448.0
    assert np.all(np.abs(d - x)[normal & ~sat] <= 2.0 ** -4 * np.abs(x)[normal & ~sat])
    assert np.all(np.abs(d - x)[~normal] <= 2.0 ** -10 * scale[~normal])
    assert np.all(np.abs(d[sat]) == 448.0 * scale[sat])
    # Every non-zero block reaches the top binade of the format.
    blk = np.abs(q.reshape(rows, 5, 32).astype(np.int64) & 0x7F).max(axis=2)
    assert np.all((blk >= 0x78) | (np.abs(x).reshape(rows, 5, 32).max(axis=2) == 0))


def test_moe_mxfp8_plumbing_equals_fp64_shard_on_dequantised_operands():
    t, hd, fe, experts, topk, e_start, e_local = 24, 64, 32, 8, 2, 2, 3
    ids = np.stack([RNG.permutation(experts)[:topk] for _ in range(t)])
    w = RNG.random((t, topk))
    x = RNG.standard_normal((t, hd))
    wgu = RNG.standard_normal((e_local, 2 * fe, hd)) * 0.2
    wd = RNG.standard_normal((e_local, hd, fe)) * 0.2
    gq, gs = zip(*[O.mx_quantize(wgu[e]) for e in range(e_local)])
    dq, ds = zip(*[O.mx_quantize(wd[e]) for e in range(e_local)])
    got = O.moe_forward_mxfp8(x, ids, w, gq, gs, dq, ds, e_start, act_round=False, act_quant=False)
    xd = O.mx_dequantize(*O.mx_quantize(x))
    wgud = np.stack([O.mx_dequantize(gq[e], gs[e]) for e in range(e_local)])
    wdd = np.stack([O.mx_dequantize(dq[e], ds[e]) for e in range(e_local)])
    want = O.moe_forward(xd, ids, w, wgud, wdd, e_start)[0]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    # With the activation quantised too, the result stays within the format's
    # error of the unquantised shard.
    full = O.moe_forward_mxfp8(x, ids, w, gq, gs, dq, ds, e_start)
    ref = O.moe_forward(x, ids, w, wgu, wd, e_start)[0]
    rel = np.linalg.norm(full - ref) / np.linalg.norm(ref)
    assert 1e-4 < rel < 0.1
