"""Python binding of libqg.so, the MI355X (gfx950) quantized GEMM library.

Argument marshalling only: torch tensors supply device pointers, torch's current
stream supplies the hipStream_t, and every step of the computation runs in the
library's HIP kernels.  The entry points mirror include/qg.h one to one:
``prepared_bytes``, ``prepare``, ``workspace_bytes``, ``gemm``, ``moe_block_m``,
``moe_capacity``, ``moe_align``, ``moe_grouped_map``, ``moe_gemm``, ``moe_swiglu``,
``moe_combine``, ``quantize_e4m3_rows``, ``quantize_e2m1_rows``, ``dequant``, ``status_str``,
``version`` and the measurement helpers ``ceiling_read`` and ``ceiling_mfma``.

There is no fallback: if libqg.so is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqg.so")

# Enumerations (values as in include/qg.h).
W_INT4, W_UINT4, W_FP4_E2M1, W_FP8_E4M3 = 1, 2, 3, 4
S_F16, S_BF16, S_F32, S_UE8M0 = 1, 2, 3, 4
A_F16, A_BF16, A_FP8_E4M3, A_FP4_E2M1 = 1, 2, 3, 4
O_F16, O_BF16 = 1, 2
C_NATIVE, C_W_TO_FP8, C_BATCH_INVARIANT = 0, 1, 4
MOE_CONTIGUOUS, MOE_MASKED = 1, 2

STATUS = {0: "QG_OK", 1: "QG_ERR_INVALID_ARG", 2: "QG_ERR_UNSUPPORTED", 3: "QG_ERR_ARCH_MISMATCH",
          4: "QG_ERR_NOT_PREPARED", 5: "QG_ERR_WORKSPACE", 6: "QG_ERR_CAPACITY", 7: "QG_ERR_HIP"}
EXPORTS = ["qg_prepared_bytes", "qg_prepare", "qg_workspace_bytes", "qg_gemm", "qg_moe_block_m", "qg_moe_capacity",
           "qg_moe_align", "qg_moe_grouped_map", "qg_moe_gemm", "qg_moe_swiglu", "qg_moe_combine",
           "qg_quantize_e4m3_rows", "qg_quantize_e2m1_rows", "qg_dequant", "qg_ceiling_read", "qg_ceiling_mfma", "qg_ceiling_lds",
           "qg_gemm_noalloc", "qg_noalloc_scratch_bytes",
           "qg_status_str", "qg_version"]


class QGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_status_text(status)})")


class LayerDesc(ctypes.Structure):
    _fields_ = [("w_type", ctypes.c_int32), ("s_type", ctypes.c_int32), ("group_k", ctypes.c_int32),
                ("has_zero", ctypes.c_int32), ("a_type", ctypes.c_int32), ("compute", ctypes.c_int32),
                ("out_type", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64)]


class Prepared(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("layout_version", ctypes.c_uint32), ("gfx_arch", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32), ("desc", LayerDesc), ("dev", ctypes.c_void_p),
                ("bytes", ctypes.c_uint64), ("off_w", ctypes.c_uint64), ("off_s", ctypes.c_uint64),
                ("off_z", ctypes.c_uint64), ("w_expert_bytes", ctypes.c_uint64), ("s_expert_bytes", ctypes.c_uint64),
                ("z_expert_bytes", ctypes.c_uint64)]


_lib = None


def lib():
    """Load libqg.so (built in-tree by quantized_gemm_amd.build); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m quantized_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        pd, pp = ctypes.POINTER(LayerDesc), ctypes.POINTER(Prepared)
        L.qg_prepared_bytes.argtypes, L.qg_prepared_bytes.restype = [pd], sz
        L.qg_prepare.argtypes, L.qg_prepare.restype = [pd, vp, vp, vp, vp, sz, pp, vp], i32
        L.qg_workspace_bytes.argtypes, L.qg_workspace_bytes.restype = [pp, i64, i32], sz
        L.qg_gemm.argtypes, L.qg_gemm.restype = [pp, vp, vp, vp, i64, vp, sz, vp], i32
        L.qg_moe_block_m.argtypes, L.qg_moe_block_m.restype = [pp, i64, i32], i32
        L.qg_moe_capacity.argtypes = [i64, i32, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.qg_moe_capacity.restype = i32
        L.qg_moe_align.argtypes = [vp, i64, i32, i32, i32, vp, i64, vp, i64, vp, vp]
        L.qg_moe_align.restype = i32
        L.qg_moe_grouped_map.argtypes = [i32, vp, i32, i64, i64, i32, vp, i64, vp, i64, vp, vp]
        L.qg_moe_grouped_map.restype = i32
        L.qg_moe_gemm.argtypes = [pp, vp, vp, vp, vp, vp, i64, i32, i32, vp, vp, sz, vp]
        L.qg_moe_gemm.restype = i32
        L.qg_moe_swiglu.argtypes, L.qg_moe_swiglu.restype = [vp, i64, i64, i32, i32, vp, vp, vp], i32
        L.qg_moe_combine.argtypes = [vp, vp, vp, i64, i32, i32, i64, i32, vp, vp]
        L.qg_moe_combine.restype = i32
        L.qg_quantize_e4m3_rows.argtypes = [vp, i64, i64, i32, vp, vp, vp]
        L.qg_quantize_e2m1_rows.argtypes, L.qg_quantize_e2m1_rows.restype = [vp, i64, i64, i32, vp, vp, vp], i32
        L.qg_quantize_e4m3_rows.restype = i32
        L.qg_dequant.argtypes, L.qg_dequant.restype = [pp, i32, vp, vp], i32
        u64 = ctypes.c_uint64
        L.qg_gemm_noalloc.argtypes, L.qg_gemm_noalloc.restype = [pp, vp, vp, vp, i64, vp], i32
        L.qg_noalloc_scratch_bytes.argtypes, L.qg_noalloc_scratch_bytes.restype = [], sz
        L.qg_ceiling_read.argtypes, L.qg_ceiling_read.restype = [vp, u64, i32, vp, u64, vp], i32
        L.qg_ceiling_mfma.argtypes, L.qg_ceiling_mfma.restype = [i32, i64, i32, vp, u64, vp], i32
        L.qg_ceiling_lds.argtypes, L.qg_ceiling_lds.restype = [i64, i32, vp, u64, vp], i32
        L.qg_status_str.argtypes, L.qg_status_str.restype = [i32], ctypes.c_char_p
        L.qg_version.argtypes, L.qg_version.restype = [], i32
        _lib = L
    return _lib


def _status_text(s: int) -> str:
    try:
        return lib().qg_status_str(s).decode()
    except Exception:  # library unavailable while formatting an error
        return "?"


def status_str(s: int) -> str:
    return lib().qg_status_str(s).decode()


def version() -> int:
    return lib().qg_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, where: str):
    if status != 0:
        raise QGError(status, where)


def make_desc(w_type, s_type, group_k, has_zero, a_type, compute, out_type, num_experts, n, k) -> LayerDesc:
    return LayerDesc(w_type, s_type, group_k, int(has_zero), a_type, compute, out_type, num_experts, n, k)


def prepared_bytes(desc: LayerDesc) -> int:
    return lib().qg_prepared_bytes(ctypes.byref(desc))


def prepare(desc: LayerDesc, w, scales, zeros, out, stream=None) -> Prepared:
    """Repack logical device tensors into ``out`` (a uint8 device tensor) and return the handle."""
    p = Prepared()
    st = lib().qg_prepare(ctypes.byref(desc), _ptr(w), _ptr(scales), _ptr(zeros), _ptr(out),
                          out.numel() * out.element_size(), ctypes.byref(p), _stream(stream))
    _check(st, "qg_prepare")
    return p


def workspace_bytes(p: Prepared, m_or_tokens: int, topk: int = 0) -> int:
    return lib().qg_workspace_bytes(ctypes.byref(p), m_or_tokens, topk)


def gemm(p: Prepared, x, x_scale, y, m: int, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().qg_gemm(ctypes.byref(p), _ptr(x), _ptr(x_scale), _ptr(y), m, _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "qg_gemm")


def gemm_call(p: Prepared, x, x_scale, y, m: int, ws=None, stream=None):
    """qg_gemm with every argument converted once: returns a no-argument callable that enqueues
    the same launch again (for timing loops, where per-call tensor slicing and stream lookup
    would cost more host time than a small kernel takes on the GPU)."""
    fn = lib().qg_gemm
    args = (ctypes.byref(p), _ptr(x), _ptr(x_scale), _ptr(y), m, _ptr(ws),
            0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))

    def call():
        st = fn(*args)
        if st != 0:
            raise QGError(st, "qg_gemm")
    return call


def gemm_noalloc(p: Prepared, x, x_scale, y, m: int, stream=None):
    """qg_gemm with the library's own per-GPU scratch array as the workspace (no allocation)."""
    st = lib().qg_gemm_noalloc(ctypes.byref(p), _ptr(x), _ptr(x_scale), _ptr(y), m, _stream(stream))
    _check(st, "qg_gemm_noalloc")


def noalloc_scratch_bytes() -> int:
    return lib().qg_noalloc_scratch_bytes()


def moe_block_m(p: Prepared, tokens: int, topk: int) -> int:
    return lib().qg_moe_block_m(ctypes.byref(p), tokens, topk)


def moe_capacity(tokens: int, topk: int, num_experts: int, block_m: int):
    cs, cb = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().qg_moe_capacity(tokens, topk, num_experts, block_m, ctypes.byref(cs), ctypes.byref(cb)),
           "qg_moe_capacity")
    return cs.value, cb.value


def moe_align(topk_ids, tokens: int, topk: int, num_experts: int, block_m: int, sorted_ids, expert_ids,
              num_post_pad, stream=None):
    st = lib().qg_moe_align(_ptr(topk_ids), tokens, topk, num_experts, block_m, _ptr(sorted_ids), sorted_ids.numel(),
                            _ptr(expert_ids), expert_ids.numel(), _ptr(num_post_pad), _stream(stream))
    _check(st, "qg_moe_align")


def moe_grouped_map(layout: int, offsets_or_counts, num_experts: int, rows_total: int, rows_per_expert: int,
                    block_m: int, sorted_ids, expert_ids, num_post_pad, stream=None):
    """Block map of a grouped-contiguous (offsets [E+1]) or grouped-masked (counts [E]) MoE input."""
    st = lib().qg_moe_grouped_map(layout, _ptr(offsets_or_counts), num_experts, rows_total, rows_per_expert, block_m,
                                  _ptr(sorted_ids), sorted_ids.numel(), _ptr(expert_ids), expert_ids.numel(),
                                  _ptr(num_post_pad), _stream(stream))
    _check(st, "qg_moe_grouped_map")


def moe_gemm(p: Prepared, x, x_scale, sorted_ids, expert_ids, num_post_pad, tokens: int, topk: int, block_m: int,
             y, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().qg_moe_gemm(ctypes.byref(p), _ptr(x), _ptr(x_scale), _ptr(sorted_ids), _ptr(expert_ids),
                           _ptr(num_post_pad), tokens, topk, block_m, _ptr(y), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "qg_moe_gemm")


def moe_gemm_call(p: Prepared, x, x_scale, sorted_ids, expert_ids, num_post_pad, tokens: int, topk: int,
                  block_m: int, y, ws=None, stream=None):
    """qg_moe_gemm with every argument converted once (see gemm_call)."""
    fn = lib().qg_moe_gemm
    args = (ctypes.byref(p), _ptr(x), _ptr(x_scale), _ptr(sorted_ids), _ptr(expert_ids), _ptr(num_post_pad), tokens,
            topk, block_m, _ptr(y), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))

    def call():
        st = fn(*args)
        if st != 0:
            raise QGError(st, "qg_moe_gemm")
    return call


def moe_swiglu(gate_up, rows: int, inter: int, in_type: int, out_type: int, out, out_scale=None, stream=None):
    """act = silu(gate) * up per row (gate = first ``inter`` columns); f16/bf16, per-row e4m3 or MXFP4 output."""
    st = lib().qg_moe_swiglu(_ptr(gate_up), rows, inter, in_type, out_type, _ptr(out), _ptr(out_scale),
                             _stream(stream))
    _check(st, "qg_moe_swiglu")


def moe_combine(y, weights, topk_ids, tokens: int, topk: int, num_experts: int, n: int, dtype: int, out,
                stream=None):
    """out[t] = sum_j weights[t, j] * y[t*topk + j] over the slots routed inside [0, E)."""
    st = lib().qg_moe_combine(_ptr(y), _ptr(weights), _ptr(topk_ids), tokens, topk, num_experts, n, dtype, _ptr(out),
                              _stream(stream))
    _check(st, "qg_moe_combine")


def quantize_e4m3_rows(x, rows: int, k: int, in_type: int, codes, scale, stream=None):
    """Per-token absmax e4m3 quantization of 16-bit rows: codes [rows][k] uint8, scale [rows] float32."""
    st = lib().qg_quantize_e4m3_rows(_ptr(x), rows, k, in_type, _ptr(codes), _ptr(scale), _stream(stream))
    _check(st, "qg_quantize_e4m3_rows")


def quantize_e2m1_rows(x, rows: int, k: int, in_type: int, codes, scales, stream=None):
    """MXFP4 quantization of 16-bit rows: codes [rows][k/2] uint8 (packed e2m1), scales [rows][k/32] uint8."""
    st = lib().qg_quantize_e2m1_rows(_ptr(x), rows, k, in_type, _ptr(codes), _ptr(scales), _stream(stream))
    _check(st, "qg_quantize_e2m1_rows")


def dequant(p: Prepared, expert: int, out, stream=None):
    _check(lib().qg_dequant(ctypes.byref(p), expert, _ptr(out), _stream(stream)), "qg_dequant")


def ceiling_read(buf, nbytes: int, loads_per_lane: int, sink, stream=None):
    """Measurement helper: one streaming read of ``nbytes`` of ``buf`` (see qg_ceiling_read)."""
    _check(lib().qg_ceiling_read(_ptr(buf), nbytes, loads_per_lane, _ptr(sink), sink.numel(), _stream(stream)),
           "qg_ceiling_read")


def ceiling_mfma(dtype: int, iters: int, workgroups: int, sink, stream=None):
    """Measurement helper: back-to-back MFMAs (dtype 0 bf16, 1 e4m3, 2 e2m1; see qg_ceiling_mfma)."""
    _check(lib().qg_ceiling_mfma(dtype, iters, workgroups, _ptr(sink), sink.numel(), _stream(stream)),
           "qg_ceiling_mfma")


def ceiling_lds(iters: int, workgroups: int, sink, stream=None):
    """Measurement helper: conflict-free 16-byte LDS reads by 8 waves per workgroup (see qg_ceiling_lds)."""
    _check(lib().qg_ceiling_lds(iters, workgroups, _ptr(sink), sink.numel(), _stream(stream)), "qg_ceiling_lds")
