"""The C ABI loads, exports every declared symbol, and rejects bad arguments on the host (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import quantized_gemm_amd as qg
from quantized_gemm_amd import layers, synth
from oracle import align as A
from oracle import layout as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "qg.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qg_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = qg.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(qg.EXPORTS)


def test_status_strings_and_version():
    for s in range(8):
        assert qg.status_str(s)
    assert qg.version() >> 16 == 1


WORKLOADS = [
    synth.dense_w4a16_sym_f16(m=1, n=64, k=256)[0],
    synth.dense_w4a16_asym_bf16(m=1, n=64, k=512)[0],
    synth.dense_w8a8_fp8(m=1, n=64, k=256)[0],
    synth.moe_w4a16_mxfp4(t=2, experts=3, topk=2, n=64, k=256)[0],
    synth.moe_w4a8_int4(t=2, experts=3, topk=2, n=64, k=256)[0],
]


@pytest.mark.parametrize("layer", WORKLOADS, ids=lambda l: l.name)
def test_prepared_bytes_matches_layout_reference(layer):
    d = layers.desc_for(layer)
    sz = L.sizes(layer.w_type, layer.s_type, layer.n, layer.k, layer.group, layer.experts, layer.z is not None)
    assert qg.prepared_bytes(d) == sz["total"]


def _desc(**kw):
    base = dict(w_type=qg.W_UINT4, s_type=qg.S_BF16, group_k=128, has_zero=1, a_type=qg.A_BF16,
                compute=qg.C_NATIVE, out_type=qg.O_BF16, num_experts=1, n=512, k=1024)
    base.update(kw)
    return qg.make_desc(**base)


@pytest.mark.parametrize("kw", [dict(n=100), dict(k=1000), dict(group_k=64), dict(has_zero=0), dict(s_type=qg.S_F32),
                                dict(w_type=qg.W_INT4), dict(a_type=qg.A_FP8_E4M3),
                                dict(w_type=qg.W_FP4_E2M1, s_type=qg.S_UE8M0, group_k=128, has_zero=0),
                                dict(w_type=qg.W_FP8_E4M3, s_type=qg.S_F32, group_k=0, has_zero=0),
                                dict(w_type=9), dict(n=-64), dict(out_type=qg.O_F16)])
def test_invalid_or_unsupported_descriptions_have_no_size(kw):
    assert qg.prepared_bytes(_desc(**kw)) == 0


def test_prepare_rejects_before_touching_the_gpu():
    lib = qg.lib()
    p = qg.Prepared()
    d = _desc()
    st = lib.qg_prepare(ctypes.byref(d), None, None, None, None, 0, ctypes.byref(p), None)
    assert st == 1  # null pointers
    st = lib.qg_prepare(ctypes.byref(_desc(k=1000)), None, None, None, None, 0, ctypes.byref(p), None)
    assert st == 2  # unsupported shape
    fake = ctypes.c_void_p(4096)
    st = lib.qg_prepare(ctypes.byref(d), fake, fake, fake, fake, 16, ctypes.byref(p), None)
    assert st == 5  # output buffer too small


def _forged(**kw):
    p = qg.Prepared()
    p.magic, p.layout_version, p.gfx_arch = qg.lib() and 0x31504751, 1, 950
    p.desc = _desc()
    p.dev = 4096
    p.bytes = qg.prepared_bytes(p.desc)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_gemm_and_moe_reject_bad_handles_and_arguments():
    lib = qg.lib()
    fake = ctypes.c_void_p(4096)
    assert lib.qg_gemm(None, fake, None, fake, 1, None, 0, None) == 1
    assert lib.qg_gemm(ctypes.byref(_forged(magic=0)), fake, None, fake, 1, None, 0, None) == 4
    assert lib.qg_gemm(ctypes.byref(_forged(layout_version=2)), fake, None, fake, 1, None, 0, None) == 4
    assert lib.qg_gemm(ctypes.byref(_forged(gfx_arch=942)), fake, None, fake, 1, None, 0, None) == 3
    assert lib.qg_gemm(ctypes.byref(_forged(bytes=16)), fake, None, fake, 1, None, 0, None) == 4
    good = _forged()
    assert lib.qg_gemm(ctypes.byref(good), fake, None, fake, -1, None, 0, None) == 1
    assert lib.qg_gemm(ctypes.byref(good), fake, None, fake, 0, None, 0, None) == 0   # M == 0 is a no-op
    assert lib.qg_gemm(ctypes.byref(good), None, None, fake, 4, None, 0, None) == 1
    assert lib.qg_gemm(ctypes.byref(good), ctypes.c_void_p(4097), None, fake, 4, None, 0, None) == 1  # misaligned
    assert lib.qg_moe_gemm(ctypes.byref(good), fake, None, fake, fake, fake, 0, 2, 16, fake, None, 0, None) == 0
    assert lib.qg_moe_gemm(ctypes.byref(good), fake, None, fake, fake, fake, 4, 2, 48, fake, None, 0, None) == 2
    assert lib.qg_dequant(ctypes.byref(good), 5, fake, None) == 1


@pytest.mark.parametrize("t,topk,e,bm", [(1, 1, 128, 16), (16, 8, 128, 16), (4096, 8, 128, 64), (3, 2, 4, 2),
                                         (8192, 6, 64, 64)])
def test_capacity_matches_oracle(t, topk, e, bm):
    assert qg.moe_capacity(t, topk, e, bm) == A.capacity(t, topk, e, bm)


def test_moe_align_rejects_on_the_host():
    lib = qg.lib()
    fake = ctypes.c_void_p(4096)
    assert lib.qg_moe_align(fake, 4, 2, 8, 12, fake, 100, fake, 10, fake, None) == 1   # block not a power of two
    assert lib.qg_moe_align(fake, 4, 2, 8, 512, fake, 100, fake, 10, fake, None) == 1  # block too large
    cs, cb = A.capacity(4, 2, 8, 4)
    assert lib.qg_moe_align(fake, 4, 2, 8, 4, fake, cs - 1, fake, cb, fake, None) == 6
    assert lib.qg_moe_align(fake, 4, 2, 8, 4, fake, cs, fake, cb - 1, fake, None) == 6
    assert lib.qg_moe_align(fake, 4, 2, 1000, 4, fake, 10 ** 6, fake, 10 ** 6, fake, None) == 2
    assert lib.qg_moe_align(None, 4, 2, 8, 4, fake, cs, fake, cb, fake, None) == 1


def test_moe_layer_steps_reject_on_the_host():
    lib = qg.lib()
    fake = ctypes.c_void_p(4096)
    # swiglu: (gate_up, rows, inter, in_type, out_type, out, out_scale, stream)
    assert lib.qg_moe_swiglu(fake, 0, 64, qg.O_BF16, qg.A_BF16, fake, None, None) == 0      # no rows: no-op
    assert lib.qg_moe_swiglu(fake, -1, 64, qg.O_BF16, qg.A_BF16, fake, None, None) == 1
    assert lib.qg_moe_swiglu(fake, 4, 0, qg.O_BF16, qg.A_BF16, fake, None, None) == 1
    assert lib.qg_moe_swiglu(fake, 4, 64, 9, qg.A_BF16, fake, None, None) == 1               # bad input type
    assert lib.qg_moe_swiglu(fake, 4, 64, qg.O_BF16, 9, fake, None, None) == 1               # bad output type
    assert lib.qg_moe_swiglu(fake, 4, 60, qg.O_BF16, qg.A_BF16, fake, None, None) == 2       # inter % 8
    assert lib.qg_moe_swiglu(fake, 4, 8200, qg.O_BF16, qg.A_FP8_E4M3, fake, fake, None) == 2  # e4m3 row too long
    assert lib.qg_moe_swiglu(None, 4, 64, qg.O_BF16, qg.A_BF16, fake, None, None) == 1
    assert lib.qg_moe_swiglu(ctypes.c_void_p(4104), 4, 64, qg.O_BF16, qg.A_BF16, fake, None, None) == 1
    assert lib.qg_moe_swiglu(fake, 4, 64, qg.O_BF16, qg.A_FP8_E4M3, fake, None, None) == 1   # scales missing
    assert lib.qg_moe_swiglu(fake, 4, 64, qg.O_BF16, qg.A_FP4_E2M1, fake, None, None) == 1   # exponents missing
    assert lib.qg_moe_swiglu(fake, 4, 48, qg.O_BF16, qg.A_FP4_E2M1, fake, fake, None) == 2   # inter % 32
    # combine: (y, weights, ids, tokens, topk, experts, n, dtype, out, stream)
    assert lib.qg_moe_combine(fake, fake, fake, 0, 2, 8, 64, qg.O_BF16, fake, None) == 0
    assert lib.qg_moe_combine(fake, fake, fake, 4, 0, 8, 64, qg.O_BF16, fake, None) == 1
    assert lib.qg_moe_combine(fake, fake, fake, 4, 2, 8, 64, 7, fake, None) == 1
    assert lib.qg_moe_combine(fake, fake, fake, 4, 2, 8, 60, qg.O_BF16, fake, None) == 2
    assert lib.qg_moe_combine(fake, None, fake, 4, 2, 8, 64, qg.O_BF16, fake, None) == 1
    assert lib.qg_moe_combine(fake, ctypes.c_void_p(4098), fake, 4, 2, 8, 64, qg.O_BF16, fake, None) == 1


def test_reduction_length_rules():
    # K must be a multiple of 128 (1408 = 11 * 128 is accepted, 1000 and 1344 are not)
    assert qg.prepared_bytes(_desc(k=1408)) > 0
    assert qg.prepared_bytes(_desc(k=1344, group_k=64)) == 0
    assert qg.prepared_bytes(_desc(k=1344, group_k=0)) == 0


def test_grouped_map_rejects_on_the_host():
    lib = qg.lib()
    fake = ctypes.c_void_p(4096)
    cs, cb = A.capacity(100, 1, 8, 16)
    assert lib.qg_moe_grouped_map(3, fake, 8, 100, 0, 16, fake, cs, fake, cb, fake, None) == 1   # bad layout
    assert lib.qg_moe_grouped_map(1, fake, 8, 100, 0, 12, fake, cs, fake, cb, fake, None) == 1   # block not 2^n
    assert lib.qg_moe_grouped_map(2, fake, 8, 100, 16, 16, fake, cs, fake, cb, fake, None) == 1  # 8 * 16 != 100
    assert lib.qg_moe_grouped_map(1, fake, 2000, 100, 0, 16, fake, cs, fake, cb, fake, None) == 2  # too many experts
    assert lib.qg_moe_grouped_map(1, fake, 8, 100, 0, 16, fake, cs - 1, fake, cb, fake, None) == 6
    assert lib.qg_moe_grouped_map(1, None, 8, 100, 0, 16, fake, cs, fake, cb, fake, None) == 1


def test_batch_invariant_flag_is_a_selector_option():
    base = qg.prepared_bytes(_desc())
    assert qg.prepared_bytes(_desc(compute=qg.C_NATIVE | qg.C_BATCH_INVARIANT)) == base
    assert qg.prepared_bytes(_desc(compute=2)) == 0
    assert qg.prepared_bytes(_desc(compute=8)) == 0


def test_block_scaled_fp8_sizes_match_layout_reference():
    layer, _ = synth.moe_w8a8_fp8_block(t=2, experts=3, topk=1, n=256, k=512, seed=1)
    d = layers.desc_for(layer)
    sz = L.sizes("e4m3", "f32", 256, 512, 128, 3, False)
    assert qg.prepared_bytes(d) == sz["total"]
    # only 128 x 128 blocks, and N a multiple of the block
    assert qg.prepared_bytes(_desc(w_type=qg.W_FP8_E4M3, s_type=qg.S_F32, group_k=256, has_zero=0,
                                   a_type=qg.A_FP8_E4M3)) == 0
    assert qg.prepared_bytes(_desc(w_type=qg.W_FP8_E4M3, s_type=qg.S_F32, group_k=128, has_zero=0,
                                   a_type=qg.A_FP8_E4M3, n=448)) == 0


def test_quantize_rows_rejects_on_the_host():
    lib = qg.lib()
    fake = ctypes.c_void_p(4096)
    assert lib.qg_quantize_e4m3_rows(fake, 0, 64, qg.A_BF16, fake, fake, None) == 0         # no rows: no-op
    assert lib.qg_quantize_e4m3_rows(fake, 4, 64, qg.A_FP8_E4M3, fake, fake, None) == 1     # input must be 16-bit
    assert lib.qg_quantize_e4m3_rows(fake, 4, 60, qg.A_BF16, fake, fake, None) == 2
    assert lib.qg_quantize_e4m3_rows(fake, 4, 8200, qg.A_BF16, fake, fake, None) == 2
    assert lib.qg_quantize_e4m3_rows(fake, 4, 64, qg.A_BF16, None, fake, None) == 1
    assert lib.qg_quantize_e4m3_rows(ctypes.c_void_p(4100), 4, 64, qg.A_BF16, fake, fake, None) == 1


def test_w4a4_descriptions():
    # MXFP4 activations pair only with MXFP4 weights (e2m1, UE8M0 per 32, no zeros, native)
    mx = dict(w_type=qg.W_FP4_E2M1, s_type=qg.S_UE8M0, group_k=32, has_zero=0, a_type=qg.A_FP4_E2M1)
    layer = synth.dense_w4a4_mxfp4(m=1, n=64, k=256)[0]
    sz = L.sizes(layer.w_type, layer.s_type, layer.n, layer.k, layer.group, layer.experts, False)
    assert qg.prepared_bytes(layers.desc_for(layer)) == sz["total"]
    assert qg.prepared_bytes(_desc(**mx)) > 0
    assert qg.prepared_bytes(_desc(**dict(mx, out_type=qg.O_F16))) > 0
    assert qg.prepared_bytes(_desc(**dict(mx, group_k=64))) == 0
    assert qg.prepared_bytes(_desc(**dict(mx, compute=qg.C_W_TO_FP8))) == 0
    assert qg.prepared_bytes(_desc(a_type=qg.A_FP4_E2M1)) == 0                      # uint4 weights
    assert qg.prepared_bytes(_desc(w_type=qg.W_FP8_E4M3, s_type=qg.S_F32, group_k=0, has_zero=0,
                                   a_type=qg.A_FP4_E2M1)) == 0
    assert qg.prepared_bytes(_desc(**dict(mx, a_type=5))) == 0


def test_quantize_e2m1_rows_rejects_on_the_host():
    lib = qg.lib()
    fake = ctypes.c_void_p(4096)
    assert lib.qg_quantize_e2m1_rows(fake, 0, 64, qg.A_BF16, fake, fake, None) == 0         # no rows: no-op
    assert lib.qg_quantize_e2m1_rows(fake, 4, 64, qg.A_FP4_E2M1, fake, fake, None) == 1     # input must be 16-bit
    assert lib.qg_quantize_e2m1_rows(fake, 4, 48, qg.A_BF16, fake, fake, None) == 2          # k % 32
    assert lib.qg_quantize_e2m1_rows(fake, 4, 64, qg.A_BF16, None, fake, None) == 1
    assert lib.qg_quantize_e2m1_rows(fake, 4, 64, qg.A_BF16, ctypes.c_void_p(4104), fake, None) == 1   # codes 16-B
    assert lib.qg_quantize_e2m1_rows(ctypes.c_void_p(4100), 4, 64, qg.A_BF16, fake, fake, None) == 1
