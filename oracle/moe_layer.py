"""Reference for the MoE layer around the grouped products, in float64.  TEST INFRASTRUCTURE ONLY.

The pages time an MoE layer as the sum of its two grouped products, the gate/up
projection and the down projection ("Humming: Fast, Flexible Kernels for Quantized
Inference", benchmark paragraph; "Humming" wiki article, "Reported performance").
They do not say what joins the two products or how the per-slot results are summed.
Readings taken here (each listed in the design notes):

* the gate/up output of one (token, slot) row is [gate | up], gate = the first N/2
  columns, up = the last N/2;
* the activation between the products is SwiGLU: act = silu(gate) * up with
  silu(g) = g / (1 + exp(-g));
* the down projection multiplies each (token, slot) row by its own expert's weights
  (the same grouped product, one input row per slot);
* the layer output of token t is the routing-weighted sum over its slots,
  out[t] = sum_j w[t, j] * Y_down[t, j], with slots routed outside [0, E) skipped;
  the routing weights are an input (the router is not part of this path).

Everything is the plain definition: no blocking, no fusion, float64 throughout.
"""
from __future__ import annotations

import numpy as np

from . import quant as Q
from . import reference as R


def silu(g) -> np.ndarray:
    """g * sigmoid(g) = g / (1 + exp(-g)) in float64 (exp overflow gives -0 for very negative g)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(gate_up) -> np.ndarray:
    """[R, 2I] -> [R, I]: silu(gate) * up, gate = columns [0, I), up = columns [I, 2I)."""
    gu = np.asarray(gate_up, dtype=np.float64)
    i = gu.shape[-1] // 2
    assert gu.shape[-1] == 2 * i
    return silu(gu[..., :i]) * gu[..., i:]


def swiglu_e4m3(gate_up):
    """SwiGLU followed by per-row absmax e4m3 quantization (the next product's FP8 activations).

    The activation is computed in float64 and rounded to float32 before the quantizer,
    which is the per-token absmax reading used for every FP8 activation here
    (scale = max|row| / 448 in float32, 1 for an all-zero row; RNE onto e4m3 after
    clamping).  Returns (float64 activation [R, I], codes uint8 [R, I], scale float32 [R]).
    """
    act = swiglu(gate_up)
    codes, scale = Q.absmax_rows(act.astype(np.float32))
    return act, codes, scale


def swiglu_mxfp4(gate_up):
    """SwiGLU, rounded to bfloat16 (the 16-bit SwiGLU output), then MXFP4-quantized per 32-block
    of each row (the W4A4 down product's activations).  Returns (codes uint8 [R, I/2],
    UE8M0 bytes uint8 [R, I/32])."""
    act = Q.round_to_bf16(swiglu(gate_up))
    return Q.mxfp4_rows(act.reshape(-1, act.shape[-1]))


def moe_layer_reference_mxfp4(gate_up_layer, down_layer, acts, weights) -> np.ndarray:
    """The W4A4 layer in float64: MXFP4 activations into the gate/up product, whose output is
    stored as bfloat16 (its declared output type, rounded to nearest even), SwiGLU rounded to
    bfloat16 and quantized to MXFP4 between the products, then down product and combine.

    Both roundings are part of the layer: the MXFP4 grid is coarse enough that leaving either
    out moves hundreds of codes and some block exponents of a 600-row layer."""
    y1 = Q.round_to_bf16(np.nan_to_num(R.moe_reference(gate_up_layer, acts)))
    t, topk, n2 = y1.shape
    codes, e8 = swiglu_mxfp4(y1.reshape(t * topk, n2))

    class _A:   # activation record in the storage form R.activations reads
        x, x_scale = codes, e8
    x2 = R.activations(_A, "e2m1").reshape(t, topk, n2 // 2)
    y2 = down_reference(down_layer, x2, acts.topk_ids)
    return combine(y2, weights, acts.topk_ids, down_layer.experts)


def combine(y_slots, weights, topk_ids, experts: int) -> np.ndarray:
    """out[t, :] = sum_j w[t, j] * y[t, j, :] over slots whose expert id is in [0, E); float64 [T, N].

    y_slots: [T, topk, N]; weights: [T, topk]; rows of skipped slots are never read (they
    may hold anything, NaN included).
    """
    y = np.asarray(y_slots, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float64)
    ids = np.asarray(topk_ids)
    t, topk, n = y.shape
    out = np.zeros((t, n), dtype=np.float64)
    for j in range(topk):
        ok = (ids[:, j] >= 0) & (ids[:, j] < experts)
        out[ok] += w[ok, j][:, None] * y[ok, j, :]
    return out


def down_reference(down_layer, act, topk_ids, a_scale=None) -> np.ndarray:
    """Y[t, j, :] = act[t, j] . W_{ids[t, j]}^T, one input row per (token, slot); [T, topk, N].

    act: float64 [T, topk, I] (already scaled if it came from FP8 codes, see a_scale);
    slots routed outside [0, E) stay NaN.
    """
    ids = np.asarray(topk_ids)
    t, topk = ids.shape
    x = np.asarray(act, dtype=np.float64)
    if a_scale is not None:
        x = x * np.asarray(a_scale, dtype=np.float64).reshape(t, topk, 1)
    y = np.full((t, topk, down_layer.n), np.nan, dtype=np.float64)
    for e in np.unique(ids[(ids >= 0) & (ids < down_layer.experts)]):
        tt, jj = np.nonzero(ids == e)
        y[tt, jj, :] = R.dense_gemm(x[tt, jj], R.dequant_layer(down_layer, int(e)))
    return y


def moe_layer_reference(gate_up_layer, down_layer, acts, weights) -> np.ndarray:
    """The whole layer in float64 with unrounded intermediates: [T, N_down].

    gate/up product (every slot) -> SwiGLU -> down product (every slot) -> weighted sum
    over slots.  The activations of the first product are what its kernel reads
    (f16/bf16 values).
    """
    y1 = R.moe_reference(gate_up_layer, acts)
    act = swiglu(y1)
    y2 = down_reference(down_layer, act, acts.topk_ids)
    return combine(y2, weights, acts.topk_ids, down_layer.experts)
