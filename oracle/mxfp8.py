"""Oracle of MXFP8 block quantisation and the MXFP8 expert shard (fp64).

Test infrastructure only (see the package docstring).  MOE-core, technical
summary 2.5 (selective precision: the router, embeddings and optimizer stay in
high precision while the expert GEMMs and their activations run in a
low-precision format; MXFP8 is one of the recipes named).

The pages name MXFP8 without defining it; the reading here is the published
OCP Microscaling (MX) format: blocks of 32 consecutive values along the
reduction dimension share one power-of-two scale stored as an 8-bit exponent
(E8M0, value 2^(byte - 127)); each value is an FP8 E4M3 number (bias 7, no
infinities, largest finite 448).  For a block with largest magnitude X the
shared exponent is floor(log2 X) - 8 (8 is the largest E4M3 exponent), clamped
to [-127, 127]; an all-zero block (or one below 2^-126) takes -127.  Each
value is divided by the scale and rounded to the nearest E4M3 value, ties to
the even code, magnitudes above 448 saturating to 448.

Scale layout (shared with the library): per row, 4 * ceil(K / 128) bytes, the
block b's exponent at byte b and the bytes past the last block set to 127.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def e4m3_value(code):
    """Value of an E4M3 code (NaN for 0x7F / 0xFF), from the format's fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp, man = (code >> 3) & 0xF, code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man / 8.0 * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


# Non-negative finite codes 0x00 .. 0x7E and their values, ascending.
_POS_CODES = np.arange(0x7F)
_POS_VALUES = np.array([e4m3_value(c) for c in _POS_CODES])


def e4m3_round(v):
    """Nearest E4M3 code of each value (ties to the even code), saturating at
    448.  Works on the magnitude over the grid of finite codes, then adds the
    sign bit (a zero result keeps the sign of a negative input: -0)."""
    v = _f64(v)
    mag = np.minimum(np.abs(v), 448.0)
    idx = np.searchsorted(_POS_VALUES, mag)  # first grid value >= mag
    idx = np.clip(idx, 0, len(_POS_VALUES) - 1)
    lo = np.clip(idx - 1, 0, len(_POS_VALUES) - 1)
    d_hi = _POS_VALUES[idx] - mag
    d_lo = mag - _POS_VALUES[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    code = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[idx]).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def shared_exponent(block_max):
    """floor(log2 X) - 8 clamped to [-127, 127]; -127 for X < 2^-126 (and 0)."""
    x = _f64(block_max)
    _, e = np.frexp(np.where(x > 0, x, 1.0))  # x = m 2^e, m in [0.5, 1)
    se = np.where(x >= 2.0 ** -126, e - 1 - 8, -127)
    return np.clip(se, -127, 127).astype(np.int64)


def scale_width(k):
    return 4 * ((k + 127) // 128)


def mx_quantize(x):
    """Rows of ``x [rows, K]`` (K a multiple of 32) to ``(codes [rows, K]
    uint8, scales [rows, scale_width(K)] uint8)``."""
    x = _f64(x)
    rows, k = x.shape
    assert k % 32 == 0
    nb = k // 32
    blocks = x.reshape(rows, nb, 32)
    se = shared_exponent(np.abs(blocks).max(axis=2))  # [rows, nb]
    codes = e4m3_round(blocks / (2.0 ** se)[:, :, None]).reshape(rows, k)
    scales = np.full((rows, scale_width(k)), 127, dtype=np.uint8)
    scales[:, :nb] = (se + 127).astype(np.uint8)
    return codes, scales


def mx_dequantize(codes, scales):
    """Values of MXFP8 rows: code value x 2^(scale byte - 127)."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, k = codes.shape
    vals = np.array([e4m3_value(c) for c in range(256)])[codes]
    se = np.asarray(scales, dtype=np.int64)[:, :k // 32] - 127
    return (vals.reshape(rows, k // 32, 32) * (2.0 ** se)[:, :, None]).reshape(rows, k)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def bf16_round(v):
    """Round values to bfloat16 (8 significant bits, exponent range of fp32),
    to the nearest representable value with ties to the even significand,
    returned as fp64.  The exact input is rounded once (no fp32 step): write
    |v| = m 2^e with m in [0.5, 1); the spacing of bf16 values there is
    2^(e-8), or 2^-133 below the smallest normal 2^-126; v / spacing is exact
    in fp64 and np.rint rounds it half to even.  A magnitude that rounds past
    the largest finite bf16, 2^128 (1 - 2^-8), becomes infinite."""
    v = _f64(v)
    _, e = np.frexp(v)
    spacing = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(v / spacing) * spacing
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)


def moe_forward_mxfp8(x, topk_ids, topk_w, w_gu_q, w_gu_s, w_d_q, w_d_s, e_start, act_round=True,
                      act_quant=True):
    """The expert shard with MXFP8 expert GEMMs: the token rows are quantised
    along the hidden dimension, the weights arrive quantised (``w_gu_q/_s``
    per expert [2Fe, Hd], ``w_d_q/_s`` per expert [Hd, Fe]); each expert
    computes ``act = silu(g) * u`` from the dequantised operands (exact
    products, fp64 sums), rounds that value once to the nearest bf16 (the
    stored activation; ``act_round``), quantises it along Fe
    (``act_quant``), and projects it down; the unpermute sums ``w[t,k] * y``
    per token (k ascending).  Returns ``out [T, Hd]``."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    tokens, topk = ids.shape
    w = _f64(topk_w)
    xq, xs = mx_quantize(x)
    xd = mx_dequantize(xq, xs)
    e_local = np.shape(w_gu_q)[0]
    y_of = {}
    for e in range(e_local):
        sel = [(t, k) for t in range(tokens) for k in range(topk) if ids[t, k] == e_start + e]
        if not sel:
            continue
        rows = np.array([t for t, _ in sel])
        wgu = mx_dequantize(w_gu_q[e], w_gu_s[e])
        fe = wgu.shape[0] // 2
        xe = xd[rows]
        act = _silu(xe @ wgu[:fe].T) * (xe @ wgu[fe:].T)
        if act_round:
            act = bf16_round(act)
        if act_quant:
            act = mx_dequantize(*mx_quantize(act))
        y = act @ mx_dequantize(w_d_q[e], w_d_s[e]).T
        for tk, yr in zip(sel, y):
            y_of[tk] = yr
    out = np.zeros_like(xd)
    for t in range(tokens):
        for k in range(topk):
            if (t, k) in y_of:
                out[t] += w[t, k] * y_of[(t, k)]
    return out
