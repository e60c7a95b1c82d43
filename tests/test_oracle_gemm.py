"""Pins for the oracle's dequantization and products (CPU only)."""
import numpy as np
import pytest

from conftest import load_golden
from oracle import align as A
from oracle import formats as F
from oracle import reference as R
from quantized_gemm_amd import synth


def _layer(w_type, a_type, s_type, n, k, group, experts, w, s, z=None, compute="native"):
    return synth.Layer("t", w_type, a_type, s_type, "bf16", n, k, group, experts, w, s, z, compute)


# ---- hand-worked fixtures ---------------------------------------------------------------

def test_fixture_uint4_zero_point():
    g = load_golden("w4a16_uint4_zero_tiny.json")
    w = np.array(g["w_u32"], dtype=np.uint32).reshape(1, 2, 1)
    s = np.array(g["scale_bf16_bits"], dtype=np.uint16).reshape(1, 2, 1)
    z = np.array(g["zeros"], dtype=np.uint8).reshape(1, 2, 1)
    lay = _layer("uint4", "bf16", "bf16", 2, 8, 8, 1, w, s, z)
    y = R.dense_gemm(np.array([g["x"]], dtype=np.float64), R.dequant_layer(lay))
    assert np.array_equal(y[0], np.array(g["y"]))


def test_fixture_int4_symmetric_two_groups():
    g = load_golden("w4a16_int4_sym_tiny.json")
    w = np.array(g["w_u32"], dtype=np.uint32).reshape(1, 1, 1)
    s = np.array(g["scale_f16_bits"], dtype=np.uint16).reshape(1, 1, 2)
    lay = _layer("int4", "f16", "f16", 1, 8, 4, 1, w, s)
    y = R.dense_gemm(np.array([g["x"]], dtype=np.float64), R.dequant_layer(lay))
    assert np.array_equal(y[0], np.array(g["y"]))


def test_fixture_mxfp4():
    g = load_golden("mxfp4_tiny.json")
    w = np.array(g["w_u8"], dtype=np.uint8).reshape(1, 1, 16)
    s = np.array(g["scale_ue8m0"], dtype=np.uint8).reshape(1, 1, 1)
    lay = _layer("e2m1", "bf16", "ue8m0", 1, 32, 32, 1, w, s)
    y = R.dense_gemm(np.array([g["x"]], dtype=np.float64), R.dequant_layer(lay))
    assert np.array_equal(y[0], np.array(g["y"]))


def test_fixture_w8a8_fp8():
    g = load_golden("w8a8_fp8_tiny.json")
    lay = _layer("e4m3", "e4m3", "f32", 1, 4, 0, 1,
                 np.array(g["w_codes"], dtype=np.uint8).reshape(1, 1, 4),
                 np.array(g["w_scale"], dtype=np.float32).reshape(1, 1, 1))
    acts = synth.Acts(np.array([g["x_codes"]], dtype=np.uint8), np.array(g["x_scale"], np.float32), None)
    y = R.dense_reference(lay, acts)
    assert np.array_equal(y[0], np.array(g["y"]))


# ---- brute force on tiny inputs: triple loops with per-element decoding ----------------

def _brute_dense(x, nib_or_codes, sv, zv, decode, group, k):
    m, n = x.shape[0], nib_or_codes.shape[0]
    y = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                g = 0 if group == 0 else kk // group
                v = decode(nib_or_codes[j, kk])
                if zv is not None:
                    v = v - zv[j, g]
                acc += x[i, kk] * v * sv[j, g]
            y[i, j] = acc
    return y


@pytest.mark.parametrize("w_type", ["int4", "uint4", "e2m1", "e4m3"])
def test_bruteforce_equals_vectorised(w_type):
    rng = np.random.default_rng(11)
    m, n, k = 3, 5, 64
    group = {"int4": 16, "uint4": 32, "e2m1": 32, "e4m3": 0}[w_type]
    ng = 1 if group == 0 else k // group
    x = rng.integers(-4, 5, size=(m, k)).astype(np.float64)   # integer-valued: every sum exact
    if w_type in ("int4", "uint4"):
        nib = rng.integers(0, 16, size=(n, k))
        w = synth.pack_nibbles_u32(nib).reshape(1, n, k // 8)
        s = synth.f32_to_bf16_bits(np.exp2(rng.integers(-3, 3, size=(1, n, ng))).astype(np.float32))
        z = rng.integers(0, 16, size=(1, n, ng)).astype(np.uint8) if w_type == "uint4" else None
        lay = _layer(w_type, "bf16", "bf16", n, k, group, 1, w, s, z)
        dec = lambda c: float(F.decode_int4(c, w_type == "int4"))
        codes = nib
        sv = F.decode_bf16(s[0])
    elif w_type == "e2m1":
        codes = rng.integers(0, 16, size=(n, k))
        w = synth.pack_nibbles_u8(codes).reshape(1, n, k // 2)
        s = rng.integers(120, 130, size=(1, n, ng)).astype(np.uint8)
        lay = _layer(w_type, "bf16", "ue8m0", n, k, group, 1, w, s)
        dec = lambda c: float(F.decode_e2m1(c))
        sv = F.decode_ue8m0(s[0]); z = None
    else:
        codes = rng.integers(0, 256, size=(n, k))
        codes[(codes & 0x7F) == 0x7F] = 0x38
        w = codes.astype(np.uint8).reshape(1, n, k)
        s = np.exp2(rng.integers(-3, 3, size=(1, n, 1))).astype(np.float32)
        lay = _layer(w_type, "e4m3", "f32", n, k, group, 1, w, s)
        dec = lambda c: float(F.decode_e4m3(c))
        sv = s[0].astype(np.float64); z = None
    zv = None if z is None else z[0].astype(np.float64)
    ref = _brute_dense(x, codes, sv, zv, dec, group, k)
    got = R.dense_gemm(x, R.dequant_layer(lay))
    assert np.array_equal(got, ref)


# ---- closed forms and special cases ------------------------------------------------------

def test_one_hot_rows_pick_out_dequantized_columns_and_ones_give_row_sums():
    layer, _ = synth.dense_w4a16_asym_bf16(m=1, n=32, k=256, seed=2)
    w = R.dequant_layer(layer)
    x = np.zeros((3, 256)); x[0, 5] = 1; x[1, 130] = 1; x[2, :] = 1
    y = R.dense_gemm(x, w)
    assert np.array_equal(y[0], w[:, 5]) and np.array_equal(y[1], w[:, 130])
    assert np.allclose(y[2], w.sum(axis=1), rtol=0, atol=1e-12)


def test_unit_scale_zero_zero_reduces_to_code_values_and_group_k_is_channel():
    rng = np.random.default_rng(4)
    n, k = 4, 64
    nib = rng.integers(0, 16, size=(n, k))
    w = synth.pack_nibbles_u32(nib).reshape(1, n, k // 8)
    one = synth.f32_to_bf16_bits(np.ones((1, n, 2), np.float32))
    lay = _layer("uint4", "bf16", "bf16", n, k, 32, 1, w, one, np.zeros((1, n, 2), np.uint8))
    assert np.array_equal(R.dequant_layer(lay), nib.astype(np.float64))
    sc = synth.f32_to_bf16_bits(rng.uniform(0.005, 0.02, (1, n, 1)).astype(np.float32))
    a = R.dequant_layer(_layer("uint4", "bf16", "bf16", n, k, k, 1, w, sc))
    b = R.dequant_layer(_layer("uint4", "bf16", "bf16", n, k, 0, 1, w, sc))
    assert np.array_equal(a, b)


def test_quantize_dequantize_roundtrip_is_exact():
    # w = (u - z) * s  =>  u = w / s + z exactly in fp64 for every code
    layer, _ = synth.dense_w4a16_asym_bf16(m=1, n=64, k=512, seed=5)
    w = R.dequant_layer(layer)
    s = np.repeat(F.decode_bf16(layer.s[0]), 128, axis=1)
    z = np.repeat(layer.z[0].astype(np.float64), 128, axis=1)
    u = F.unpack_u32_nibbles(layer.w[0]).astype(np.float64)
    assert np.array_equal(w / s + z, u)
    layer, _ = synth.dense_w4a16_sym_f16(m=1, n=64, k=512, seed=6)
    w = R.dequant_layer(layer)
    s = np.repeat(F.decode_f16(layer.s[0]), 128, axis=1)
    q = F.decode_int4(F.unpack_u32_nibbles(layer.w[0]), True)
    assert np.array_equal(w / s, q)


def test_sign_and_orientation_of_product():
    # a transposed operand or a wrong sign would break this asymmetric case
    layer, acts = synth.dense_w4a16_sym_f16(m=2, n=16, k=128, seed=9)
    w = R.dequant_layer(layer)
    x = R.activations(acts, "f16")
    y = R.dense_reference(layer, acts)
    assert y.shape == (2, 16)
    assert y[1, 3] == pytest.approx(float(np.dot(x[1], w[3])), rel=1e-15, abs=1e-15)
    assert y[0, 7] == pytest.approx(sum(x[0, kk] * w[7, kk] for kk in range(128)), rel=1e-14, abs=1e-14)


# ---- MoE --------------------------------------------------------------------------------

def test_moe_single_expert_equals_dense_and_slices_equal_dense_on_gathered_rows():
    layer, acts = synth.moe_w4a16_mxfp4(t=6, experts=4, topk=2, n=32, k=64, seed=1)
    y = R.moe_reference(layer, acts)
    x = R.activations(acts, "bf16")
    for e in range(4):
        tt, jj = np.nonzero(acts.topk_ids == e)
        if tt.size:
            ref = R.dense_gemm(x[tt], R.dequant_layer(layer, e))
            assert np.array_equal(y[tt, jj], ref)
    one = synth.Acts(acts.x, None, np.zeros((6, 1), np.int32))
    y1 = R.moe_reference(layer, one)
    assert np.array_equal(y1[:, 0], R.dense_gemm(x, R.dequant_layer(layer, 0)))


def test_moe_token_permutation_permutes_rows_and_invalid_ids_stay_unwritten():
    layer, acts = synth.moe_w4a8_int4(t=8, experts=4, topk=2, n=32, k=128, seed=2)
    y = R.moe_reference(layer, acts)
    p = np.random.default_rng(0).permutation(8)
    acts_p = synth.Acts(acts.x[p], acts.x_scale[p], acts.topk_ids[p])
    assert np.array_equal(R.moe_reference(layer, acts_p), y[p])
    ids = acts.topk_ids.copy(); ids[3, 1] = -1; ids[5, 0] = 99
    y2 = R.moe_reference(layer, synth.Acts(acts.x, acts.x_scale, ids))
    assert np.all(np.isnan(y2[3, 1])) and np.all(np.isnan(y2[5, 0]))
    assert np.array_equal(y2[0], y[0])


def test_moe_w4a8_matches_explicit_scale_factorisation():
    # Y = sx[t] * sum_k e4m3(xq[t,k]) * q[e,n,k] * s[e,n,k/128]
    layer, acts = synth.moe_w4a8_int4(t=3, experts=2, topk=1, n=16, k=256, seed=3)
    y = R.moe_reference(layer, acts)
    for t in range(3):
        e = acts.topk_ids[t, 0]
        q = F.decode_int4(F.unpack_u32_nibbles(layer.w[e]), True)
        s = F.decode_bf16(layer.s[e])
        xv = F.decode_e4m3(acts.x[t])
        ref = np.array([sum(float(acts.x_scale[t]) * np.dot(xv[g*128:(g+1)*128], q[n_, g*128:(g+1)*128]) * s[n_, g]
                            for g in range(2)) for n_ in range(16)])
        assert np.allclose(y[t, 0], ref, rtol=1e-13, atol=1e-13)


# ---- e2m1 weights x e4m3 activations (W4A8 MXFP4) ----------------------------------------

def test_w4a8_mxfp4_brute_force_is_exact():
    # every product e2m1 * 2^(E-127) * e4m3 * 2^j is exact in float64, and so is the sum of a
    # few of them: the vectorised oracle must equal per-element decoding and triple loops
    layer, acts = synth.dense_w4a8_mxfp4(m=3, n=16, k=64, seed=4)
    acts.x_scale = np.array([0.5, 2.0, 0.25], np.float32)          # powers of two: exact
    y = R.dense_reference(layer, acts)
    nib = F.unpack_u8_nibbles(layer.w[0])
    e8 = layer.s[0].astype(np.int64)
    ref = np.zeros((3, 16))
    for m in range(3):
        for n in range(16):
            for k in range(64):
                w = float(F.decode_e2m1(nib[n, k])) * 2.0 ** (int(e8[n, k // 32]) - 127)
                ref[m, n] += float(F.decode_e4m3(acts.x[m, k])) * float(acts.x_scale[m]) * w
    assert np.array_equal(y, ref)


def test_w4a8_mxfp4_reduces_to_w4a16_mxfp4_on_the_same_values():
    # every e4m3 value is a bf16 value: with scale 1 the same activations written as bf16 give
    # exactly the same oracle product
    layer, acts = synth.dense_w4a8_mxfp4(m=4, n=32, k=256, seed=5)
    acts.x_scale = np.ones(4, np.float32)
    x16 = synth.f32_to_bf16_bits(F.decode_e4m3(acts.x).astype(np.float32))
    l16 = synth.Layer("t", "e2m1", "bf16", "ue8m0", "bf16", 32, 256, 32, 1, layer.w, layer.s, None)
    assert np.array_equal(R.dense_reference(layer, acts), R.dense_reference(l16, synth.Acts(x16, None, None)))


# ---- block-scaled e4m3 (scales over 128 x 128 weight blocks and 1 x 128 activation groups) ----

def test_block_scaled_brute_force_is_exact():
    layer, acts = synth.dense_w8a8_fp8_block(m=3, n=256, k=256, seed=6)
    rng = np.random.default_rng(6)
    layer.s = (2.0 ** rng.integers(-9, -4, size=layer.s.shape)).astype(np.float32)   # powers of two: exact
    acts.x_scale = (2.0 ** rng.integers(-3, 2, size=acts.x_scale.shape)).astype(np.float32)
    y = R.dense_reference(layer, acts)
    wv = F.decode_e4m3(layer.w[0])
    xv = F.decode_e4m3(acts.x)
    ref = np.zeros((3, 256))
    for m in range(3):
        for n in range(256):
            for k in range(256):
                ref[m, n] += (xv[m, k] * float(acts.x_scale[m, k // 128])) * (wv[n, k] * float(layer.s[0, n // 128, k // 128]))
    assert np.array_equal(y, ref)


def test_block_scaled_uniform_scales_reduce_to_channel_scales():
    layer, acts = synth.dense_w8a8_fp8_block(m=4, n=256, k=384, seed=7)
    layer.s = np.full(layer.s.shape, 0.0078125, np.float32)
    acts.x_scale = np.repeat(np.array([[0.5], [0.25], [2.0], [1.0]], np.float32), 3, axis=1)
    ch = synth.Layer("t", "e4m3", "e4m3", "f32", "bf16", 256, 384, 0, 1, layer.w, np.full((1, 256, 1), 0.0078125, np.float32), None)
    ych = R.dense_reference(ch, synth.Acts(acts.x, acts.x_scale[:, 0].copy(), None))
    assert np.array_equal(R.dense_reference(layer, acts), ych)


def test_block_quantizer_scales_each_block_by_its_own_absmax():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((256, 384)).astype(np.float32)
    x[:128, 128:256] *= 100.0                                 # one loud block
    q, s = synth.absmax_e4m3_blocks(x, 128, 128)
    for bi in range(2):
        for bj in range(3):
            blk = x[128 * bi:128 * (bi + 1), 128 * bj:128 * (bj + 1)]
            assert s[bi, bj] == np.float32(np.max(np.abs(blk)) / np.float32(448.0))
            qb = F.decode_e4m3(q[128 * bi:128 * (bi + 1), 128 * bj:128 * (bj + 1)])
            assert np.max(np.abs(qb)) == 448.0
            assert np.max(np.abs(qb * float(s[bi, bj]) - blk)) <= 2.0 ** -4 * np.max(np.abs(blk)) + 1e-6
