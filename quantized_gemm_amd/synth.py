"""Seeded synthetic inputs for the quantized GEMM workloads.

This module only *draws* inputs: random codes, scales, zero points, activations and
routing choices, in the storage formats the library consumes (raw bit patterns in
integer arrays).  It contains none of the GEMM arithmetic: no dequantization, no
products, no sums.  Both the product path (tests and the benchmark upload these
arrays to the GPU) and the CPU oracle (which decodes the same bits itself) consume
what it returns.

Storage formats produced (all row-major numpy arrays):

* int4 / uint4 weights: ``uint32 [E, N, K/8]``; element (n, k) sits in bits
  ``4*(k % 8) .. 4*(k % 8)+3`` of word ``[n, k // 8]`` (low nibble first).  Signed
  int4 is stored as the two's-complement nibble.
* e2m1 weights: ``uint8 [E, N, K/2]``; even k in the low nibble.
* e4m3 (OCP "fn" flavour) weights / activations: ``uint8`` codes.
* f16 / bf16 values: ``uint16`` bit patterns.
* UE8M0 scales: ``uint8`` biased exponents.
* zero points: ``uint8 [E, N, K/G]`` holding 0..15.
* routing: ``int32 [T, topk]`` expert ids.

The value distributions and shapes follow the five benchmark workloads: dense
W4A16 (symmetric fp16 and asymmetric bf16), dense W8A8 FP8, MoE W4A16 with MXFP4
weights and MoE W4A8 with int4 weights under a skewed router.  Draw order inside
one workload is fixed: activations, codes, scales, zeros, routing logits.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_MAX = 448.0


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 (torch's cast), returned as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> float16, returned as uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> OCP e4m3 codes (torch's cast). Input must already be clamped."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def absmax_e4m3_rows(x: np.ndarray):
    """Per-row absmax quantization to e4m3 (input generation for the FP8 workloads).

    scale = max|row| / 448 in float32 (1.0 for an all-zero row); code = RNE_e4m3(clamp(x / scale)).
    Returns (codes uint8 [R, C], scale float32 [R]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    q = (x / scale[:, None]).astype(np.float32)
    q = np.clip(q, -E4M3_MAX, E4M3_MAX)
    return f32_to_e4m3_codes(q), scale


def pack_nibbles_u32(nib: np.ndarray) -> np.ndarray:
    """[.., K] values 0..15 -> uint32 [.., K/8], element k at bits 4*(k%8) (low nibble first).

    Packs byte pairs (even k low) and reads four bytes as one little-endian word, which
    puts element k at bits 4*(k%8); no wider-than-byte temporaries (full-size MoE layers
    hold billions of codes)."""
    nib = np.asarray(nib)
    *lead, k = nib.shape
    assert k % 8 == 0
    b = np.ascontiguousarray(pack_nibbles_u8(nib.astype(np.uint8, copy=False)))
    return b.view("<u4").reshape(*lead, k // 8)


def random_nibbles_u32(rng: np.random.Generator, lead: tuple, k: int) -> np.ndarray:
    """Uniform 4-bit codes, packed like pack_nibbles_u32: [*lead, K/8] uint32.

    A uniform random byte is two independent uniform nibbles (element 2j low, 2j+1 high),
    so the bytes are drawn directly; read as two's complement a nibble is uniform over
    [-8, 7], as an unsigned code uniform over [0, 15]."""
    assert k % 8 == 0
    b = rng.integers(0, 256, size=(*lead, k // 2), dtype=np.uint8)
    return b.view("<u4").reshape(*lead, k // 8)


def pack_nibbles_u8(nib: np.ndarray) -> np.ndarray:
    """[.., K] values 0..15 -> uint8 [.., K/2], even k in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    *lead, k = nib.shape
    assert k % 2 == 0
    v = nib.reshape(*lead, k // 2, 2)
    return (v[..., 0] | (v[..., 1] << 4)).astype(np.uint8)


def topk_from_logits(logits: np.ndarray, topk: int) -> np.ndarray:
    """Top-k expert ids by descending logit (softmax is monotone, so this is softmax top-k).

    Ties go to the lower expert id (stable sort).  Slot order is descending logit.
    """
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :topk].astype(np.int32)


def router_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over all experts (float32) taken at the chosen ids, not renormalized: [T, topk].

    The router sits before the hot path; its probabilities are an input of the combine step."""
    l = np.asarray(logits, dtype=np.float32)
    e = np.exp(l - np.max(l, axis=1, keepdims=True)).astype(np.float32)
    p = (e / np.sum(e, axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1).astype(np.float32)


@dataclass
class Layer:
    """One quantized layer in storage form plus its activations."""
    name: str
    w_type: str            # "int4" | "uint4" | "e2m1" | "e4m3"
    a_type: str            # "f16" | "bf16" | "e4m3" | "e2m1"
    s_type: str            # "f16" | "bf16" | "f32" | "ue8m0"
    out_type: str          # "f16" | "bf16"
    n: int
    k: int
    group: int             # 0 = per output channel
    experts: int
    w: np.ndarray          # packed codes, see module doc
    s: np.ndarray          # scales: uint16 bits / float32 / uint8 exponents, [E, N, G]
    z: np.ndarray | None   # uint8 [E, N, G] or None
    compute: str = "native"  # "native" | "w_to_fp8"
    meta: dict = field(default_factory=dict)


@dataclass
class Acts:
    x: np.ndarray                  # uint16 bits [M, K] (f16/bf16), uint8 e4m3 codes [M, K] or packed e2m1 [M, K/2]
    x_scale: np.ndarray | None     # float32 [M] (or [M, K/128]) for e4m3, uint8 UE8M0 [M, K/32] for e2m1
    topk_ids: np.ndarray | None    # int32 [T, topk] for MoE
    topk_weights: np.ndarray | None = None   # float32 [T, topk]: router probabilities of the chosen experts


# ---------------------------------------------------------------------------
# Workloads.  Names describe what they are; sizes are arguments.
# ---------------------------------------------------------------------------

def dense_w4a16_sym_f16(m: int = 16, n: int = 512, k: int = 1024, group: int = 128, seed: int = 0):
    """Dense W4A16, symmetric int4 in [-8, 7], fp16 group scales in [0.005, 0.02], fp16 activations."""
    rng = _rng(seed)
    x = f32_to_f16_bits(rng.standard_normal((m, k), dtype=np.float32))
    w = random_nibbles_u32(rng, (1, n), k)          # two's complement codes: q uniform in [-8, 7]
    ng = 1 if group == 0 else k // group            # group 0: one scale per output channel
    s = f32_to_f16_bits(rng.uniform(0.005, 0.02, size=(1, n, ng)).astype(np.float32))
    layer = Layer("dense_w4a16_sym_f16", "int4", "f16", "f16", "f16", n, k, group, 1, w, s, None)
    return layer, Acts(x, None, None)


def dense_w4a16_asym_bf16(m: int = 16, n: int = 8192, k: int = 8192, group: int = 128, seed: int = 0):
    """Dense W4A16, uint4 codes in [0, 15] with uint4 zero points in [6, 9], bf16 group scales."""
    rng = _rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    w = random_nibbles_u32(rng, (1, n), k)          # u uniform in [0, 15]
    ng = 1 if group == 0 else k // group            # group 0: one scale per output channel
    s = f32_to_bf16_bits(rng.uniform(0.005, 0.02, size=(1, n, ng)).astype(np.float32))
    z = rng.integers(6, 10, size=(1, n, ng), dtype=np.uint8)
    layer = Layer("dense_w4a16_asym_bf16", "uint4", "bf16", "bf16", "bf16", n, k, group, 1, w, s, z)
    return layer, Acts(x, None, None)


def dense_w8a8_fp8(m: int = 1, n: int = 7168, k: int = 7168, seed: int = 0):
    """Dense W8A8: per-token absmax e4m3 activations, per-channel absmax e4m3 weights (N(0, 0.02))."""
    rng = _rng(seed)
    xq, sx = absmax_e4m3_rows(rng.standard_normal((m, k), dtype=np.float32))
    wf = (rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    wq, sw = absmax_e4m3_rows(wf)
    layer = Layer("dense_w8a8_fp8", "e4m3", "e4m3", "f32", "bf16", n, k, 0, 1,
                  wq.reshape(1, n, k), sw.reshape(1, n, 1), None)
    return layer, Acts(xq, sx, None)


def absmax_e4m3_blocks(x: np.ndarray, br: int, bc: int):
    """Absmax e4m3 quantization per br x bc block of a 2-D array (rows, columns divisible):
    returns (codes uint8 like x, scales float32 [R/br, C/bc]); each block quantized like one
    row of absmax_e4m3_rows."""
    r, c = x.shape
    blocks = np.asarray(x, np.float32).reshape(r // br, br, c // bc, bc).transpose(0, 2, 1, 3).reshape(-1, br * bc)
    q, sc = absmax_e4m3_rows(blocks)
    q = q.reshape(r // br, c // bc, br, bc).transpose(0, 2, 1, 3).reshape(r, c)
    return np.ascontiguousarray(q), sc.reshape(r // br, c // bc)


def dense_w8a8_fp8_block(m: int = 16, n: int = 7168, k: int = 7168, block: int = 128, seed: int = 0):
    """Dense W8A8 with block scales: e4m3 weights of N(0, 0.02) quantized per block x block tile
    (absmax, float32 scales [N/block, K/block]); e4m3 activations of N(0,1) rows quantized per
    (row, block of K) (float32 scales [M, K/block])."""
    rng = _rng(seed)
    xq, sx = absmax_e4m3_blocks(rng.standard_normal((m, k), dtype=np.float32), 1, block)
    wf = (rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    wq, sw = absmax_e4m3_blocks(wf, block, block)
    layer = Layer("dense_w8a8_fp8_block", "e4m3", "e4m3", "f32", "bf16", n, k, block, 1,
                  wq.reshape(1, n, k), sw.reshape(1, n // block, k // block), None)
    return layer, Acts(xq, sx, None)


def moe_w8a8_fp8_block(t: int = 16, experts: int = 8, topk: int = 2, n: int = 256, k: int = 512, block: int = 128,
                       seed: int = 0):
    """MoE W8A8 with block scales (as dense_w8a8_fp8_block, per expert), softmax top-k routing of
    N(0,1) logits."""
    rng = _rng(seed)
    xq, sx = absmax_e4m3_blocks(rng.standard_normal((t, k), dtype=np.float32), 1, block)
    ws, ss = [], []
    for _ in range(experts):
        wf = (rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
        q, sc = absmax_e4m3_blocks(wf, block, block)
        ws.append(q)
        ss.append(sc)
    logits = rng.standard_normal((t, experts), dtype=np.float32)
    ids = topk_from_logits(logits, topk)
    layer = Layer("moe_w8a8_fp8_block", "e4m3", "e4m3", "f32", "bf16", n, k, block, experts,
                  np.stack(ws), np.stack(ss), None)
    return layer, Acts(xq, sx, ids, router_weights(logits, ids))


def moe_w8a8_fp8(t: int = 16, experts: int = 8, topk: int = 2, n: int = 256, k: int = 512, seed: int = 0):
    """MoE W8A8: per-token absmax e4m3 activations, per-(expert, channel) absmax e4m3 weights
    (N(0, 0.02)), softmax top-k routing of N(0,1) logits."""
    rng = _rng(seed)
    xq, sx = absmax_e4m3_rows(rng.standard_normal((t, k), dtype=np.float32))
    wf = (rng.standard_normal((experts * n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    wq, sw = absmax_e4m3_rows(wf)
    logits = rng.standard_normal((t, experts), dtype=np.float32)
    ids = topk_from_logits(logits, topk)
    layer = Layer("moe_w8a8_fp8", "e4m3", "e4m3", "f32", "bf16", n, k, 0, experts,
                  wq.reshape(experts, n, k), sw.reshape(experts, n, 1), None)
    return layer, Acts(xq, sx, ids, router_weights(logits, ids))


def moe_w4a16_mxfp4(t: int = 16, experts: int = 128, topk: int = 8, n: int = 4096, k: int = 7168,
                    seed: int = 0):
    """MoE W4A16 with MXFP4 weights: e2m1 codes uniform over all 16 codes, UE8M0 exponents 119..123
    per 32 elements along K, bf16 activations, softmax top-k routing of N(0,1) logits."""
    rng = _rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((t, k), dtype=np.float32))
    w = rng.integers(0, 256, size=(experts, n, k // 2), dtype=np.uint8)
    s = (127 + rng.integers(-8, -3, size=(experts, n, k // 32), dtype=np.int64)).astype(np.uint8)
    logits = rng.standard_normal((t, experts), dtype=np.float32)
    ids = topk_from_logits(logits, topk)
    layer = Layer("moe_w4a16_mxfp4", "e2m1", "bf16", "ue8m0", "bf16", n, k, 32, experts, w, s, None)
    return layer, Acts(x, None, ids, router_weights(logits, ids))


def dense_w4a8_mxfp4(m: int = 16, n: int = 4096, k: int = 7168, out: str = "bf16", seed: int = 0):
    """Dense W4A8 with MXFP4 weights: e2m1 codes uniform over all 16 codes, UE8M0 exponents 119..123
    per 32 elements along K, per-token absmax e4m3 activations of N(0,1) rows."""
    rng = _rng(seed)
    xq, sx = absmax_e4m3_rows(rng.standard_normal((m, k), dtype=np.float32))
    w = rng.integers(0, 256, size=(1, n, k // 2), dtype=np.uint8)
    s = (127 + rng.integers(-8, -3, size=(1, n, k // 32), dtype=np.int64)).astype(np.uint8)
    layer = Layer("dense_w4a8_mxfp4", "e2m1", "e4m3", "ue8m0", out, n, k, 32, 1, w, s, None)
    return layer, Acts(xq, sx, None)


def moe_w4a8_mxfp4(t: int = 16, experts: int = 128, topk: int = 8, n: int = 4096, k: int = 7168, seed: int = 0):
    """MoE W4A8 with MXFP4 weights (the MXFP4 workload's weights and routing with per-token absmax e4m3
    activations instead of bf16): e2m1 codes uniform, UE8M0 exponents 119..123 per 32 along K, softmax
    top-k routing of N(0,1) logits."""
    rng = _rng(seed)
    xq, sx = absmax_e4m3_rows(rng.standard_normal((t, k), dtype=np.float32))
    w = rng.integers(0, 256, size=(experts, n, k // 2), dtype=np.uint8)
    s = (127 + rng.integers(-8, -3, size=(experts, n, k // 32), dtype=np.int64)).astype(np.uint8)
    logits = rng.standard_normal((t, experts), dtype=np.float32)
    ids = topk_from_logits(logits, topk)
    layer = Layer("moe_w4a8_mxfp4", "e2m1", "e4m3", "ue8m0", "bf16", n, k, 32, experts, w, s, None)
    return layer, Acts(xq, sx, ids, router_weights(logits, ids))


def mxfp4_act_codes(rng, rows: int, k: int):
    """Random MXFP4 activations as stored: packed e2m1 codes (every byte value equally likely) and
    UE8M0 exponents 124..130 per 32 elements of a row."""
    x = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    xs = (127 + rng.integers(-3, 4, size=(rows, k // 32), dtype=np.int64)).astype(np.uint8)
    return x, xs


def dense_w4a4_mxfp4(m: int = 16, n: int = 4096, k: int = 7168, out: str = "bf16", seed: int = 0):
    """Dense W4A4 MXFP4: e2m1 weights with UE8M0 exponents 119..123 per 32 along K (as the W4A8
    MXFP4 workload) times MXFP4 activations (random codes, exponents 124..130 per 32)."""
    rng = _rng(seed)
    w = rng.integers(0, 256, size=(1, n, k // 2), dtype=np.uint8)
    s = (127 + rng.integers(-8, -3, size=(1, n, k // 32), dtype=np.int64)).astype(np.uint8)
    x, xs = mxfp4_act_codes(rng, m, k)
    layer = Layer("dense_w4a4_mxfp4", "e2m1", "e2m1", "ue8m0", out, n, k, 32, 1, w, s, None)
    return layer, Acts(x, xs, None)


def moe_w4a4_mxfp4(t: int = 16, experts: int = 128, topk: int = 8, n: int = 4096, k: int = 7168, seed: int = 0):
    """MoE W4A4 MXFP4: the MXFP4 MoE workload's weights and routing with MXFP4 activations."""
    rng = _rng(seed)
    w = rng.integers(0, 256, size=(experts, n, k // 2), dtype=np.uint8)
    s = (127 + rng.integers(-8, -3, size=(experts, n, k // 32), dtype=np.int64)).astype(np.uint8)
    x, xs = mxfp4_act_codes(rng, t, k)
    logits = rng.standard_normal((t, experts), dtype=np.float32)
    ids = topk_from_logits(logits, topk)
    layer = Layer("moe_w4a4_mxfp4", "e2m1", "e2m1", "ue8m0", "bf16", n, k, 32, experts, w, s, None)
    return layer, Acts(x, xs, ids, router_weights(logits, ids))


def moe_w4a8_int4(t: int = 64, experts: int = 64, topk: int = 6, n: int = 2816, k: int = 4096,
                  group: int = 128, hot_frac: float = 0.2, hot_experts=(0, 1, 2, 3), hot_bias: float = 3.0,
                  seed: int = 0):
    """MoE W4A8: symmetric int4 weights in [-8, 7] with bf16 group-128 scales (converted to e4m3 inside
    the kernel), per-token absmax e4m3 activations, and a skewed router: a seeded 20% of tokens get
    +3.0 on the logits of four hot experts before top-k."""
    rng = _rng(seed)
    xq, sx = absmax_e4m3_rows(rng.standard_normal((t, k), dtype=np.float32))
    w = random_nibbles_u32(rng, (experts, n), k)    # two's complement codes: q uniform in [-8, 7]
    ng = 1 if group == 0 else k // group            # group 0: one scale per output channel
    s = f32_to_bf16_bits(rng.uniform(0.005, 0.02, size=(experts, n, ng)).astype(np.float32))
    logits = rng.standard_normal((t, experts), dtype=np.float32)
    n_hot = int(round(hot_frac * t))
    hot_tokens = rng.permutation(t)[:n_hot]
    for e in hot_experts:
        if e < experts:
            logits[hot_tokens, e] += np.float32(hot_bias)
    ids = topk_from_logits(logits, topk)
    layer = Layer("moe_w4a8_int4", "int4", "e4m3", "bf16", "bf16", n, k, group, experts, w, s, None,
                  compute="w_to_fp8")
    return layer, Acts(xq, sx, ids, router_weights(logits, ids))


# ---------------------------------------------------------------------------
# The rest of an MoE layer: the down projection's weights and standalone inputs of the
# steps between and after the two grouped products.  Drawn from their own seeds, so the
# gate/up workloads above keep their draws.
# ---------------------------------------------------------------------------

def moe_down_mxfp4(experts: int = 128, n: int = 7168, k: int = 2048, seed: int = 100):
    """Down projection with MXFP4 weights (K = half the gate/up width): e2m1 codes uniform over all
    16 codes, UE8M0 exponents 119..123 per 32 elements along K, bf16 activations and output."""
    rng = _rng(seed)
    w = rng.integers(0, 256, size=(experts, n, k // 2), dtype=np.uint8)
    s = (127 + rng.integers(-8, -3, size=(experts, n, k // 32), dtype=np.int64)).astype(np.uint8)
    return Layer("moe_down_mxfp4", "e2m1", "bf16", "ue8m0", "bf16", n, k, 32, experts, w, s, None)


def moe_down_w4a8(experts: int = 64, n: int = 4096, k: int = 1408, group: int = 128, seed: int = 100):
    """Down projection of the W4A8 layer: symmetric int4 in [-8, 7], bf16 group scales in
    [0.005, 0.02], per-row e4m3 activations (the SwiGLU output quantized per row)."""
    rng = _rng(seed)
    w = random_nibbles_u32(rng, (experts, n), k)
    ng = 1 if group == 0 else k // group
    s = f32_to_bf16_bits(rng.uniform(0.005, 0.02, size=(experts, n, ng)).astype(np.float32))
    return Layer("moe_down_w4a8", "int4", "e4m3", "bf16", "bf16", n, k, group, experts, w, s, None,
                 compute="w_to_fp8")


def moe_down_w4a8_mxfp4(experts: int = 128, n: int = 7168, k: int = 2048, seed: int = 100):
    """Down projection of the W4A8 MXFP4 layer: MXFP4 weights drawn like moe_down_mxfp4, e4m3
    activations (the SwiGLU output quantized per row)."""
    layer = moe_down_mxfp4(experts=experts, n=n, k=k, seed=seed)
    layer.name, layer.a_type = "moe_down_w4a8_mxfp4", "e4m3"
    return layer


def moe_down_w4a4_mxfp4(experts: int = 128, n: int = 7168, k: int = 2048, seed: int = 100):
    """Down projection of the W4A4 MXFP4 layer: MXFP4 weights drawn like moe_down_mxfp4, MXFP4
    activations (the SwiGLU output quantized per 32-block)."""
    layer = moe_down_mxfp4(experts=experts, n=n, k=k, seed=seed)
    layer.name, layer.a_type = "moe_down_w4a4_mxfp4", "e2m1"
    return layer


def gate_up_values(rows: int, inter: int, dtype: str = "bf16", sigma: float = 4.0, seed: int = 0):
    """Gate/up rows [rows, 2*inter] as f16/bf16 bits: N(0, sigma) values plus a few exact specials
    (0, +-1, +-20, +-100) in the gate half of the first row (saturation of the sigmoid)."""
    rng = _rng(seed)
    v = (rng.standard_normal((rows, 2 * inter), dtype=np.float32) * np.float32(sigma)).astype(np.float32)
    sp = np.array([0.0, 1.0, -1.0, 20.0, -20.0, 100.0, -100.0], dtype=np.float32)
    if rows > 0:
        v[0, :min(inter, sp.size)] = sp[:min(inter, sp.size)]
    return f32_to_bf16_bits(v) if dtype == "bf16" else f32_to_f16_bits(v)


def act_rows(rows: int, k: int, dtype: str = "bf16", sigma: float = 4.0, seed: int = 0):
    """Activation rows of a down product, [rows, k]: N(0, sigma) as f16/bf16 bits, or per-row absmax
    e4m3 codes + float32 scales (dtype "e4m3")."""
    rng = _rng(seed)
    v = (rng.standard_normal((rows, k), dtype=np.float32) * np.float32(sigma)).astype(np.float32)
    if dtype == "e4m3":
        return absmax_e4m3_rows(v)
    return (f32_to_bf16_bits(v) if dtype == "bf16" else f32_to_f16_bits(v)), None


def slot_outputs(tokens: int, topk: int, n: int, experts: int, dtype: str = "bf16", drop_frac: float = 0.0,
                 seed: int = 0):
    """Inputs of the combine step: per-(token, slot) rows [T*topk, N] (f16/bf16 bits, N(0, 4)),
    router probabilities [T, topk] (softmax of N(0,1) logits at the top-k ids) and the ids, a
    seeded fraction of slots set to -1 (dropped)."""
    rng = _rng(seed)
    y = f32_to_bf16_bits if dtype == "bf16" else f32_to_f16_bits
    vals = y((rng.standard_normal((tokens * topk, n), dtype=np.float32) * np.float32(4.0)).astype(np.float32))
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    ids = topk_from_logits(logits, topk)
    w = router_weights(logits, ids)
    if drop_frac > 0:
        drop = rng.random((tokens, topk)) < drop_frac
        ids = np.where(drop, -1, ids).astype(np.int32)
    return vals, w, ids


WORKLOADS = {
    "dense_w4a16_sym_f16": dense_w4a16_sym_f16,
    "dense_w4a16_asym_bf16": dense_w4a16_asym_bf16,
    "dense_w8a8_fp8": dense_w8a8_fp8,
    "moe_w4a16_mxfp4": moe_w4a16_mxfp4,
    "moe_w4a8_int4": moe_w4a8_int4,
    "dense_w4a8_mxfp4": dense_w4a8_mxfp4,
    "moe_w4a8_mxfp4": moe_w4a8_mxfp4,
    "dense_w8a8_fp8_block": dense_w8a8_fp8_block,
    "dense_w4a4_mxfp4": dense_w4a4_mxfp4,
    "moe_w4a4_mxfp4": moe_w4a4_mxfp4,
}
