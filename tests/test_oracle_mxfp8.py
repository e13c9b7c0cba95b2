"""Pins for the oracle's MXFP8 pieces (CPU only).

The E4M3 decode of all 256 codes and the round-to-nearest-even encode against
PyTorch's independent float8_e4m3fn conversion (below 464, where that
conversion does not turn to NaN); saturation above 448; the shared exponent
against its closed form on exact powers of two; exact round trips of values
already on the MX grid; the per-element error bound of the format; the bf16
rounding of the stored activation against PyTorch's float32 -> bfloat16
conversion (fp32 inputs: random, ties,
subnormals, extremes) and, for fp64 inputs, against the nearest-neighbour
definition; and the MXFP8 expert shard, with the activation's rounding and
quantisation off, against the fp64 shard on the dequantised operands and, with
both on, against the same steps built from PyTorch's bf16 conversion
(MOE-core, technical summary 2.5: expert GEMMs in low precision, router and
weights' master copies high precision).
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


def _torch_bf16(v32):
    """fp32 values -> bfloat16 by PyTorch's conversion (round to nearest even),
    back to fp64."""
    return torch.from_numpy(np.asarray(v32, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def test_bf16_round_matches_torch_on_fp32_inputs():
    """For inputs that are fp32 values one rounding is one rounding: the
    oracle must agree with torch bit for bit, including exact ties (the
    midpoint between two bf16 neighbours goes to the even significand),
    subnormals, the largest finite values and overflow to infinity."""
    u = RNG.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]                      # no inf / NaN inputs
    ties = (RNG.integers(0, 2 ** 16, 4000, dtype=np.uint64).astype(np.uint32) << 16) | np.uint32(0x8000)
    ties = ties[((ties >> 23) & 0xFF) != 0xFF]
    near = (RNG.integers(0, 2 ** 16, 4000, dtype=np.uint64).astype(np.uint32) << 16) | \
        RNG.choice(np.array([0x7FFF, 0x8001, 0x0001, 0xFFFF], dtype=np.uint32), 4000)
    near = near[((near >> 23) & 0xFF) != 0xFF]
    special = np.array([0x00000001, 0x00008000, 0x00018000, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F7F8000,
                        0x7F7F7FFF, 0x80000001, 0xFF7FFFFF, 0x3F808000, 0x3F818000, 0, 0x80000000], dtype=np.uint32)
    v32 = np.concatenate([u, ties, near, special]).view(np.float32)
    got = O.bf16_round(v32.astype(np.float64))
    want = _torch_bf16(v32)
    assert np.array_equal(got, want)  # infinities compare equal, no NaN inputs
    assert np.isinf(got[-9]) and np.isinf(got[-5])          # 0x7F7FFFFF and 0xFF7FFFFF round past the top
    assert got[-7] == 2.0 ** 128 * (1 - 2.0 ** -8)           # 0x7F7F7FFF stays at the largest finite bf16
    assert got[-4] == 1.0 and got[-3] == 1.015625           # ties to the even significand


def test_bf16_round_is_nearest_on_fp64_inputs():
    """Inputs with more than fp32's 24 bits: the result is a bf16 value (its
    fp32 image has 16 zero low bits) and no other bf16 value is nearer; on an
    exact tie the significand is even.  (Rounding through fp32 first would
    fail this on the values placed just off a bf16 midpoint.)"""
    base = RNG.standard_normal(20000) * 2.0 ** RNG.integers(-140, 120, 20000)
    b32 = _torch_bf16(base.astype(np.float32)).astype(np.float32)
    mid = (b32.view(np.uint32) + np.uint32(0x8000)).view(np.float32).astype(np.float64)  # exact bf16 midpoints
    off = mid * (1 + RNG.choice([-1.0, 1.0], mid.size) * 2.0 ** -30)    # just off them (below fp32 resolution)
    v = np.concatenate([base, mid, off])
    v = v[np.abs(v) < 2.0 ** 127]
    r = O.bf16_round(v)
    r32 = r.astype(np.float32)
    assert np.array_equal(r32.astype(np.float64), r)
    assert np.all((r32.view(np.uint32) & 0xFFFF) == 0)
    bits = r32.view(np.uint32)
    up = (bits + np.uint32(0x10000)).view(np.float32).astype(np.float64)   # next bf16 away from zero
    down = np.where((bits & 0x7FFFFFFF) == 0, -up,
                    (bits - np.uint32(0x10000)).view(np.float32).astype(np.float64))
    d = np.abs(v - r)
    assert np.all(d <= np.abs(v - up)) and np.all(d <= np.abs(v - down))
    tie = (d == np.abs(v - up)) | (d == np.abs(v - down))
    assert np.all(((bits[tie] >> 16) & 1) == 0)
    # the off-midpoint values differ from a round through fp32 on some inputs
    via32 = _torch_bf16(off.astype(np.float32))
    assert np.any(O.bf16_round(off) != via32)


def test_moe_mxfp8_full_path_against_torch_built_steps():
    """moe_forward_mxfp8 with the activation rounded and quantised, against
    the same steps assembled here: SwiGLU on the dequantised operands in
    fp64, PyTorch's bf16 conversion of the activation, the MX block
    quantiser, the down projection and the weighted per-token sum.  The
    activation values are fp64; torch converts them through fp32 (two
    roundings), so the data is checked first to hold no value where that
    differs from one rounding."""
    t, hd, fe, experts, topk, e_start, e_local = 20, 64, 64, 6, 2, 1, 3
    ids = np.stack([RNG.permutation(experts)[:topk] for _ in range(t)])
    w = RNG.random((t, topk))
    x = RNG.standard_normal((t, hd))
    wgu = RNG.standard_normal((e_local, 2 * fe, hd)) * 0.2
    wd = RNG.standard_normal((e_local, hd, fe)) * 0.2
    gq, gs = zip(*[O.mx_quantize(wgu[e]) for e in range(e_local)])
    dq, ds = zip(*[O.mx_quantize(wd[e]) for e in range(e_local)])
    got = O.moe_forward_mxfp8(x, ids, w, gq, gs, dq, ds, e_start)
    xd = torch.from_numpy(O.mx_dequantize(*O.mx_quantize(x)))
    want = torch.zeros((t, hd), dtype=torch.float64)
    for e in range(e_local):
        g = torch.from_numpy(O.mx_dequantize(gq[e], gs[e]))
        dw = torch.from_numpy(O.mx_dequantize(dq[e], ds[e]))
        for tok in range(t):
            for k in range(topk):
                if ids[tok, k] != e_start + e:
                    continue
                h = g @ xd[tok]
                act = torch.nn.functional.silu(h[:fe]) * h[fe:]
                assert torch.equal(act.to(torch.bfloat16).double(),
                                   torch.from_numpy(O.bf16_round(act.numpy())))  # no double-rounding case here
                a = act.to(torch.bfloat16).double().numpy()[None, :]
                aq = torch.from_numpy(O.mx_dequantize(*O.mx_quantize(a))[0])
                want[tok] += w[tok, k] * (dw @ aq)
    assert np.allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)
    # A truncating rounding of the activation would be caught: it changes the result.
    assert not np.allclose(got, O.moe_forward_mxfp8(x, ids, w, gq, gs, dq, ds, e_start, act_round=False),
                           rtol=1e-12, atol=1e-12)
