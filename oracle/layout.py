"""Reference for the prepared-weight byte layout (format version 1).  TEST INFRASTRUCTURE ONLY.

"Humming: Fast, Flexible Kernels for Quantized Inference" (standard-format paragraphs)
and "Humming" (wiki article, "Quantization representation" and "Kernel configuration
and compilation"): preprocessing repacks weights, scales and zero points into a
layout suited to the target kernel; the transformed layer is tied to its target
architecture; storage parameters need a re-transform while tuning choices may vary
per call.  The layout itself is this library's own definition, written out here
from its specification (not from the library's code):

Regions, each starting at a 256-byte aligned offset: W, then S, then Z (if zero points).

W: 16-byte units indexed [e][nb = n/16][ku = k/KU][c = n%16], KU = 32 for 4-bit
   formats and 16 for e4m3; unit byte offset = ((e*NB + nb)*KUN + ku)*256 + c*16.
   4-bit unit: four little-endian u32 words; word j holds elements k = ku*32 + 8j + i,
   i = 0..7, nibble position p holding element i = ORDER[p]:
     "pair"    [0, 2, 4, 6, 1, 3, 5, 7]  int4/uint4 with f16/bf16 activations
     "quad"    [0, 4, 1, 5, 2, 6, 3, 7]  int4 converted to e4m3 in-kernel
     "natural" [0, 1, 2, 3, 4, 5, 6, 7]  e2m1
   Nibble value: uint4 -> u; int4 with f16/bf16 activations -> c ^ 8 (biased to q + 8);
   int4 for the e4m3 conversion -> c (two's complement); e2m1 -> c.
   e4m3 unit: 16 bytes, element k = ku*16 + i at byte i.
S: elements [e][nb][g][c] = scale[e][nb*16 + c][g] in the scale type's own bytes
   (2 for f16/bf16, 4 for f32, 1 for UE8M0); channel scales have G = 1.  Block scales of
   e4m3 weights (one per G x G block of output channels x K): [e][n/G][g] as given.
Z: for each [e][nb][g] two u32 words; column c at word c/8, nibble c%8.
"""
from __future__ import annotations

import numpy as np

ORDERS = {
    "pair": [0, 2, 4, 6, 1, 3, 5, 7],
    "quad": [0, 4, 1, 5, 2, 6, 3, 7],
    "natural": [0, 1, 2, 3, 4, 5, 6, 7],
}
SCALE_BYTES = {"f16": 2, "bf16": 2, "f32": 4, "ue8m0": 1}


def _align(x: int, a: int = 256) -> int:
    return (x + a - 1) // a * a


def order_for(w_type: str, a_type: str) -> str | None:
    if w_type == "e2m1":
        return "natural"
    if w_type in ("int4", "uint4"):
        return "quad" if a_type == "e4m3" else "pair"
    return None


def sizes(w_type, s_type, n, k, group, experts, has_zero):
    bits = 8 if w_type == "e4m3" else 4
    g = 1 if group == 0 else k // group
    wb = experts * n * k * bits // 8
    block = w_type == "e4m3" and group > 0          # block scales [e][n/G][k/G], stored as given
    sb = experts * (n // group if block else n) * g * SCALE_BYTES[s_type]
    zb = experts * (n // 16) * g * 8 if has_zero else 0
    off_s = _align(wb)
    off_z = off_s + _align(sb)
    total = off_z + _align(zb)
    return dict(w_bytes=wb, s_bytes=sb, z_bytes=zb, off_w=0, off_s=off_s, off_z=off_z, total=total, groups=g)


def _logical_nibbles(layer) -> np.ndarray:
    """[E, N, K] nibble codes in the logical (unpermuted) order."""
    w = np.asarray(layer.w)
    if layer.w_type == "e2m1":
        lo = w & 0xF
        hi = w >> 4
        return np.stack([lo, hi], axis=-1).reshape(w.shape[0], w.shape[1], -1).astype(np.uint8)
    parts = [((w >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.uint8) for i in range(8)]
    return np.stack(parts, axis=-1).reshape(w.shape[0], w.shape[1], -1)


def repack(layer) -> np.ndarray:
    """Logical layer -> prepared byte image (uint8 [total])."""
    e_, n, k = layer.experts, layer.n, layer.k
    assert n % 16 == 0
    has_zero = layer.z is not None
    sz = sizes(layer.w_type, layer.s_type, n, k, layer.group, e_, has_zero)
    out = np.zeros(sz["total"], dtype=np.uint8)
    nb = n // 16
    if layer.w_type == "e4m3":
        kun = k // 16
        codes = np.asarray(layer.w, dtype=np.uint8).reshape(e_, nb, 16, kun, 16)   # e, nb, c, ku, i
        units = codes.transpose(0, 1, 3, 2, 4)                                      # e, nb, ku, c, i
        out[:sz["w_bytes"]] = units.reshape(-1)
    else:
        order = ORDERS[order_for(layer.w_type, layer.a_type)]
        nib = _logical_nibbles(layer).astype(np.uint32)
        if layer.w_type == "int4" and layer.a_type != "e4m3":
            nib = nib ^ 8
        kun = k // 32
        v = nib.reshape(e_, nb, 16, kun, 4, 8)       # e, nb, c, ku, j, i
        words = np.zeros(v.shape[:-1], dtype=np.uint32)
        for p in range(8):
            words |= v[..., order[p]] << np.uint32(4 * p)
        units = words.transpose(0, 1, 3, 2, 4)       # e, nb, ku, c, j
        out[:sz["w_bytes"]] = np.ascontiguousarray(units).astype("<u4").view(np.uint8).reshape(-1)
    # scales: [e][nb][g][c] (block scales: [e][n/G][g] as given)
    g = sz["groups"]
    s = np.asarray(layer.s)
    if layer.w_type == "e4m3" and layer.group > 0:
        s = s.reshape(e_, n // layer.group, g)
    else:
        s = s.reshape(e_, nb, 16, g).transpose(0, 1, 3, 2)
    sdt = {"f16": "<u2", "bf16": "<u2", "f32": "<f4", "ue8m0": "u1"}[layer.s_type]
    out[sz["off_s"]:sz["off_s"] + sz["s_bytes"]] = np.ascontiguousarray(s).astype(sdt).view(np.uint8).reshape(-1)
    if has_zero:
        z = np.asarray(layer.z, dtype=np.uint32).reshape(e_, nb, 16, g).transpose(0, 1, 3, 2)  # e, nb, g, c
        z = z.reshape(e_, nb, g, 2, 8)
        words = np.zeros((e_, nb, g, 2), dtype=np.uint32)
        for p in range(8):
            words |= z[..., p] << np.uint32(4 * p)
        out[sz["off_z"]:sz["off_z"] + sz["z_bytes"]] = words.astype("<u4").view(np.uint8).reshape(-1)
    return out


def unpack(buf, w_type, a_type, s_type, n, k, group, experts, has_zero):
    """Prepared byte image -> (w, s, z) in the logical storage formats (inverse of ``repack``)."""
    buf = np.asarray(buf, dtype=np.uint8)
    sz = sizes(w_type, s_type, n, k, group, experts, has_zero)
    nb = n // 16
    wbytes = buf[:sz["w_bytes"]]
    if w_type == "e4m3":
        kun = k // 16
        u = wbytes.reshape(experts, nb, kun, 16, 16).transpose(0, 1, 3, 2, 4)
        w = np.ascontiguousarray(u).reshape(experts, n, k)
    else:
        order = ORDERS[order_for(w_type, a_type)]
        kun = k // 32
        words = wbytes.view("<u4").reshape(experts, nb, kun, 16, 4).transpose(0, 1, 3, 2, 4)  # e, nb, c, ku, j
        v = np.zeros((experts, nb, 16, kun, 4, 8), dtype=np.uint32)
        for p in range(8):
            v[..., order[p]] = (words >> np.uint32(4 * p)) & np.uint32(0xF)
        if w_type == "int4" and a_type != "e4m3":
            v = v ^ 8
        nib = v.reshape(experts, n, k)
        if w_type == "e2m1":
            pairs = nib.reshape(experts, n, k // 2, 2)
            w = (pairs[..., 0] | (pairs[..., 1] << 4)).astype(np.uint8)
        else:
            r = nib.reshape(experts, n, k // 8, 8)
            w = np.zeros((experts, n, k // 8), dtype=np.uint32)
            for i in range(8):
                w |= r[..., i] << np.uint32(4 * i)
    g = sz["groups"]
    sdt = {"f16": "<u2", "bf16": "<u2", "f32": "<f4", "ue8m0": "u1"}[s_type]
    if w_type == "e4m3" and group > 0:
        s = buf[sz["off_s"]:sz["off_s"] + sz["s_bytes"]].view(sdt).reshape(experts, n // group, g).copy()
    else:
        sb = buf[sz["off_s"]:sz["off_s"] + sz["s_bytes"]].view(sdt).reshape(experts, nb, g, 16)
        s = np.ascontiguousarray(sb.transpose(0, 1, 3, 2)).reshape(experts, n, g)
    z = None
    if has_zero:
        zw = buf[sz["off_z"]:sz["off_z"] + sz["z_bytes"]].view("<u4").reshape(experts, nb, g, 2)
        zz = np.zeros((experts, nb, g, 2, 8), dtype=np.uint8)
        for p in range(8):
            zz[..., p] = (zw >> np.uint32(4 * p)) & np.uint32(0xF)
        z = np.ascontiguousarray(zz.reshape(experts, nb, g, 16).transpose(0, 1, 3, 2)).reshape(experts, n, g)
    return w, s, z
