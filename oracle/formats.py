"""Value decoders for the storage formats, written from the formats' bit-field definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the types only ("Humming" README, "Key Features": scale types BF16,
FP16, E4M3, E5M2, UE8M0; "Support Matrix": e5m10, e8m7, e4m3, e5m2, e2m1 notation).
The bit layouts are the public ones:

* int4: two's-complement nibble, value c - 16*[c >= 8]; uint4: value c.
* e2m1 (OCP MX FP4): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
  exponent 0 is subnormal (value m * 0.5).  No Inf/NaN.
* e4m3 (OCP FP8 "fn"): sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
  exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no Inf.
* UE8M0 (OCP MX scale): 2^(b - 127); b = 255 is NaN.
* f16 / bf16: IEEE binary16 / the top half of binary32.

Every decoder returns float64 and is exact.  The 4- and 8-bit decoders evaluate their
bit-field formula once for every code of the format and then index that table with the
input codes: the same values as evaluating the formula per element, far faster on the
hundreds of millions of codes of a full-size MoE layer.
"""
from __future__ import annotations

import numpy as np


def _int4_value(c, signed: bool) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64) & 0xF
    if signed:
        return np.where(c >= 8, c - 16, c).astype(np.float64)
    return c.astype(np.float64)


def _e2m1_value(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m * 0.5) * np.exp2(e - 1.0))
    return sign * mag


def _e4m3_value(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64) & 0xFF
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * np.exp2(-9.0), (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def _ue8m0_value(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64) & 0xFF
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


_TABLES = {
    "int4": _int4_value(np.arange(16), True),
    "uint4": _int4_value(np.arange(16), False),
    "e2m1": _e2m1_value(np.arange(16)),
    "e4m3": _e4m3_value(np.arange(256)),
    "ue8m0": _ue8m0_value(np.arange(256)),
}


def _lookup(name: str, c, mask: int) -> np.ndarray:
    c = np.asarray(c)
    idx = c & mask if c.dtype.kind in "ui" else np.asarray(c, dtype=np.int64) & mask
    return _TABLES[name][idx]


def decode_int4(c, signed: bool) -> np.ndarray:
    return _lookup("int4" if signed else "uint4", c, 0xF)


def decode_e2m1(c) -> np.ndarray:
    return _lookup("e2m1", c, 0xF)


def decode_e4m3(c) -> np.ndarray:
    return _lookup("e4m3", c, 0xFF)


def decode_ue8m0(b) -> np.ndarray:
    return _lookup("ue8m0", b, 0xFF)


def decode_bf16(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint32) & 0xFFFF
    return (bits << np.uint32(16)).astype(np.uint32).view(np.float32).astype(np.float64)


def decode_f16(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_scale(s, s_type: str) -> np.ndarray:
    if s_type == "f16":
        return decode_f16(s)
    if s_type == "bf16":
        return decode_bf16(s)
    if s_type == "f32":
        return np.asarray(s, dtype=np.float32).astype(np.float64)
    if s_type == "ue8m0":
        return decode_ue8m0(s)
    raise ValueError(s_type)


def decode_act(x, a_type: str) -> np.ndarray:
    if a_type == "f16":
        return decode_f16(x)
    if a_type == "bf16":
        return decode_bf16(x)
    if a_type == "e4m3":
        return decode_e4m3(x)
    if a_type == "e2m1":                       # packed codes [.., K/2], even k in the low nibble
        return decode_e2m1(unpack_u8_nibbles(x))
    raise ValueError(a_type)


def unpack_u32_nibbles(words) -> np.ndarray:
    """uint32 [.., K/8] -> [.., K] nibbles; element k at bits 4*(k%8) of word k//8."""
    w = np.asarray(words, dtype=np.uint32)
    out = np.empty(w.shape + (8,), dtype=np.uint8)
    for i in range(8):
        out[..., i] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    return out.reshape(*w.shape[:-1], w.shape[-1] * 8)


def unpack_u8_nibbles(b) -> np.ndarray:
    """uint8 [.., K/2] -> [.., K] nibbles; even k in the low nibble."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape + (2,), dtype=np.uint8)
    out[..., 0] = b & 0xF
    out[..., 1] = b >> 4
    return out.reshape(*b.shape[:-1], b.shape[-1] * 2)
