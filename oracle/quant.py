"""Reference absmax e4m3 quantizer, for pinning the synthetic FP8 inputs.  TEST INFRASTRUCTURE ONLY.

The FP8 workloads quantize activations per token and weights per output channel by
absmax ("Humming" wiki article, "Reported performance": tokenwise FP8 activations;
the workload definitions fix per-token / per-channel absmax).  The pages give no
formula; the reading used is: scale = max|row| / 448 in float32 (1 for an all-zero
row), code = round-to-nearest-even onto the e4m3 value set of clamp(x / scale, +-448).

Rounding here is done by searching the 254 finite e4m3 values (nearest value; on a
tie, the code with an even mantissa), independent of any library cast.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_e4m3


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
