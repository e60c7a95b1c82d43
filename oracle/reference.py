"""Reference dequantization and products in float64.  TEST INFRASTRUCTURE ONLY.

What the hot path computes is Y = X . dequant(Wq, scales, zeros)^T, as a dense layer
and as an MoE grouped product over routed tokens.  The method reaches exactly this
plain result (up to rounding order), so the oracle is that definition written out:
unpack the codes, decode them to float64, apply scales and zero points, multiply with
``numpy.matmul`` in float64.  No blocking, no fusion, no reordering.

Passages followed:
* "Humming: Fast, Flexible Kernels for Quantized Inference", the standard-format
  paragraphs: weights, scales and zero points are separate parameters; groupwise
  INT4 weights can pair with BF16 activations.
* "Humming" (wiki article), "Quantization representation": channel scales (one per
  output channel), group scales (a channel divided along the reduction dimension),
  optional zero points, an expert dimension for MoE.
* "Humming" (wiki article), "Device and workload selection": the indexed MoE path
  gathers input rows through routing indices.
* "Humming" (README), "Usage Example": the quantized layer output is compared with
  ``inputs.matmul(weight.T)``.

Readings where the pages are silent (each listed in the design notes):
* zero points are integers in the code domain: w = (u - z) * s;
* symmetric int4 keeps -8;
* activations are what the kernel reads: f16/bf16 values, or sx[m] * e4m3(code) (with block
  scales sx[m, k / 128] * e4m3(code)), or MXFP4 activations 2^(b[m, k / 32] - 127) * e2m1(code)
  (one UE8M0 exponent per 32 consecutive K of a row, as for MXFP4 weights);
* block scales ("Humming" wiki article, "Quantization representation": a scale shared across
  both matrix dimensions): e4m3 weights with group G > 0 carry one scale per G x G block of
  (output channel, K);
* MoE output is [T, topk, N], one row per (token, slot); routing probabilities are
  not applied; slots whose id is outside [0, E) are left unwritten (NaN here).
"""
from __future__ import annotations

import numpy as np

from . import formats as F


def dequant_codes(layer_w, layer_s, layer_z, w_type: str, s_type: str, group: int, k: int) -> np.ndarray:
    """Dequantize ONE expert's weights to float64 [N, K].

    layer_w: packed codes for one expert (uint32 [N, K/8] for int4/uint4, uint8 [N, K/2] for e2m1,
    uint8 [N, K] for e4m3); layer_s: [N, G]; layer_z: [N, G] uint8 or None.
    """
    if w_type in ("int4", "uint4"):
        codes = F.unpack_u32_nibbles(layer_w)
        vals = F.decode_int4(codes, signed=(w_type == "int4"))
    elif w_type == "e2m1":
        vals = F.decode_e2m1(F.unpack_u8_nibbles(layer_w))
    elif w_type == "e4m3":
        vals = F.decode_e4m3(layer_w)
    else:
        raise ValueError(w_type)
    n = vals.shape[0]
    assert vals.shape[1] == k
    g = k if group == 0 else group
    ngroups = k // g
    s = F.decode_scale(layer_s, s_type).reshape(n, ngroups)
    s_full = np.repeat(s, g, axis=1)
    if layer_z is not None:
        z = np.asarray(layer_z, dtype=np.int64).reshape(n, ngroups).astype(np.float64)
        vals = vals - np.repeat(z, g, axis=1)
    return vals * s_full


def is_block_scaled(layer) -> bool:
    """e4m3 weights with group > 0: one scale per group x group block of (output channel, K)."""
    return layer.w_type == "e4m3" and layer.group > 0


def _scale_rows(layer, expert: int, rows=None):
    """Scales of the given output channels as [rows, G] (block scales repeat over the block's rows)."""
    s = np.asarray(layer.s[expert])
    if is_block_scaled(layer):
        r = np.arange(layer.n) if rows is None else np.asarray(rows)
        return s[r // layer.group]
    return s if rows is None else s[np.asarray(rows)]


def dequant_layer(layer, expert: int = 0) -> np.ndarray:
    z = None if layer.z is None else layer.z[expert]
    return dequant_codes(layer.w[expert], _scale_rows(layer, expert), z, layer.w_type, layer.s_type, layer.group,
                         layer.k)


def dequant_rows(layer, expert: int, rows) -> np.ndarray:
    """Dequantize only output channels ``rows`` of one expert (for sampled checks at full size)."""
    rows = np.asarray(rows)
    z = None if layer.z is None else layer.z[expert][rows]
    return dequant_codes(layer.w[expert][rows], _scale_rows(layer, expert, rows), z,
                         layer.w_type, layer.s_type, layer.group, layer.k)


def activations(acts, a_type: str) -> np.ndarray:
    """The activation values the kernel multiplies, in float64 [M, K]."""
    x = F.decode_act(acts.x, a_type)
    if a_type == "e2m1":
        sx = F.decode_ue8m0(acts.x_scale)        # [M, K / 32]
        return x * np.repeat(sx, 32, axis=1)
    if a_type == "e4m3":
        sx = np.asarray(acts.x_scale, dtype=np.float32).astype(np.float64)
        if sx.ndim == 2:                       # one scale per (row, group of K / G columns)
            x = x * np.repeat(sx, x.shape[1] // sx.shape[1], axis=1)
        else:
            x = x * sx[:, None]
    return x


def dense_gemm(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Y[m, n] = sum_k x[m, k] * w[n, k] in float64, unrounded."""
    return np.matmul(x, w.T)


def dense_reference(layer, acts) -> np.ndarray:
    return dense_gemm(activations(acts, layer.a_type), dequant_layer(layer, 0))


def moe_reference(layer, acts, experts=None) -> np.ndarray:
    """Y[t, j, :] = X[t] . W_{ids[t, j]}^T for every (token, slot); [T, topk, N] float64.

    Each expert is dequantized on the fly (all experts at once would not fit in memory at the
    largest sizes).  Slots routed outside [0, E) stay NaN.  ``experts`` optionally restricts
    which experts are evaluated (other rows stay NaN).
    """
    x = activations(acts, layer.a_type)
    ids = np.asarray(acts.topk_ids)
    t, topk = ids.shape
    y = np.full((t, topk, layer.n), np.nan, dtype=np.float64)
    used = np.unique(ids[(ids >= 0) & (ids < layer.experts)])
    for e in used:
        if experts is not None and e not in experts:
            continue
        tt, jj = np.nonzero(ids == e)
        w = dequant_layer(layer, int(e))
        y[tt, jj, :] = dense_gemm(x[tt], w)
    return y


def relative_error(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    """max|Y - Y_ref| / max|Y_ref| over the whole tensor; non-finite GPU output counts as infinite."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    if not np.all(np.isfinite(y_gpu)):
        return float("inf")
    denom = np.max(np.abs(y_ref))
    return float(np.max(np.abs(y_gpu - y_ref)) / denom)
