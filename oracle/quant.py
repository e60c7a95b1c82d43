"""Reference absmax e4m3 quantizer, for pinning the synthetic FP8 inputs.  TEST INFRASTRUCTURE ONLY.

The FP8 workloads quantize activations per token and weights per output channel by
absmax ("Humming" wiki article, "Reported performance": tokenwise FP8 activations;
the workload definitions fix per-token / per-channel absmax).  The pages give no
formula; the reading used is: scale = max|row| / 448 in float32 (1 for an all-zero
row), code = round-to-nearest-even onto the e4m3 value set of clamp(x / scale, +-448).

Rounding here is done by searching the 254 finite e4m3 values (nearest value; on a
tie, the code with an even mantissa), independent of any library cast.

MXFP4 activations (W4A4: "Humming" README, "Key Features", lists FP4 activations; the
wiki article, "Quantization representation", names UE8M0 scales) are quantized per
block of 32 consecutive K of a row.  The pages give no rule; the reading used is the
OCP Microscaling (MX) v1.0 conversion: shared exponent E = floor(log2(max |block|)) - 2
(2 = the largest e2m1 exponent), clamped to [-127, 127], stored as the UE8M0 byte E + 127
(byte 0 for an all-zero block); each element becomes the e2m1 value nearest to
x / 2^E (ties to the even code, values above 6 saturate to 6); a code is negative only
when its magnitude is not zero.  Inputs must be finite.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_e2m1, decode_e4m3


def _table():
    codes = np.arange(256)
    vals = decode_e4m3(codes)
    finite = np.isfinite(vals)
    return codes[finite], vals[finite]


_CODES, _VALS = _table()
_POS = _VALS >= 0
_PCODES = _CODES[_POS & ~((_CODES == 0x80))]
_PVALS = _VALS[_POS & ~((_CODES == 0x80))]
_ORD = np.argsort(_PVALS)
_PCODES = _PCODES[_ORD]
_PVALS = _PVALS[_ORD]


def round_to_e4m3(x) -> np.ndarray:
    """Nearest-even e4m3 code for each |x| <= 448 (sign kept; -0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    assert np.all(a <= 448.0)
    idx = np.searchsorted(_PVALS, a)            # first value >= a
    idx = np.clip(idx, 1, _PVALS.size - 1)
    lo, hi = _PVALS[idx - 1], _PVALS[idx]
    clo, chi = _PCODES[idx - 1], _PCODES[idx]
    d_lo, d_hi = a - lo, hi - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((chi & 1) == 0))
    code = np.where(a == 0, 0, np.where(pick_hi, chi, clo))
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def absmax_rows(x):
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    q = np.clip((x32 / scale[:, None]).astype(np.float32), -448.0, 448.0)
    return round_to_e4m3(q.astype(np.float64)), scale


# the 8 non-negative e2m1 values, codes 0..7 in ascending order
_E2M1 = decode_e2m1(np.arange(8))


def round_to_e2m1(q) -> np.ndarray:
    """Nearest e2m1 code (ties to the even code, saturating at 6) for each float64 q."""
    q = np.asarray(q, dtype=np.float64)
    a = np.minimum(np.abs(q), 6.0)
    idx = np.clip(np.searchsorted(_E2M1, a), 1, 7)      # first value >= a
    lo, hi = _E2M1[idx - 1], _E2M1[idx]
    d_lo, d_hi = a - lo, hi - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (idx % 2 == 0))
    mag = np.where(a == 0, 0, np.where(pick_hi, idx, idx - 1)).astype(np.int64)
    return np.where((q < 0) & (mag != 0), mag | 8, mag).astype(np.uint8)


def mxfp4_rows(x):
    """x [M, K] (K % 32 == 0, finite) -> (packed e2m1 codes uint8 [M, K/2], UE8M0 bytes uint8 [M, K/32])."""
    x = np.asarray(x, dtype=np.float64)
    m, k = x.shape
    blocks = x.reshape(m, k // 32, 32)
    amax = np.max(np.abs(blocks), axis=2)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))           # amax = f * 2^e, f in [0.5, 1)
    shared = np.clip(e - 1 - 2, -127, 127)
    shared = np.where(amax > 0, shared, -127)
    q = blocks / np.exp2(shared)[:, :, None]
    codes = round_to_e2m1(q).reshape(m, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (shared + 127).astype(np.uint8)


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each finite float64 x, as float64.

    bfloat16 keeps 8 significant bits: the spacing at |x| in [2^e, 2^(e+1)) is 2^(e-7), and
    2^-133 below 2^-126 (subnormals); x / spacing is rounded half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(np.where(a > 0, a, 1.0))             # a = f * 2^e, f in [0.5, 1)
    spacing = np.exp2(np.maximum(e - 1, -126) - 7)
    return np.where(a > 0, np.round(x / spacing) * spacing, x)
