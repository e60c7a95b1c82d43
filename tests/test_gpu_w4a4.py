"""GPU parity of W4A4 MXFP4 (e2m1 weights and e2m1 activations, UE8M0 exponents per 32 K on
both sides) and of the MXFP4 activation quantizer, through the C ABI.

The product runs on the scaled fp4 x fp4 MFMA with both operands as stored: 16-, 32- and
64-row workgroups with K split over waves, 128 x 128 tiles, and the MFMA kernel's 128- and
256-row tiles (activations through LDS).  Every product of two scaled
e2m1 values is exact in float32, so the only roundings are the float32 accumulation and the
output conversion: bar max|Y - Y_ref| / max|Y_ref| <= 2^-8 (twice the bf16 unit roundoff).
The quantizer is compared byte for byte with the oracle's (codes and exponents).
"""
import numpy as np
import pytest
import torch

import quantized_gemm_amd as qg
from quantized_gemm_amd import layers, synth
from oracle import formats as F
from oracle import layout as L
from oracle import quant as Q
from oracle import reference as R

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qg.lib()
    yield


def test_prepare_and_readback_are_bit_exact():
    layer, _ = synth.moe_w4a4_mxfp4(t=4, experts=3, topk=2, n=128, k=512, seed=1)
    p, buf = layers.prepare_layer(layer)
    assert np.array_equal(buf.cpu().numpy(), L.repack(layer))
    for e in range(layer.experts):
        out = torch.empty((layer.n, layer.k), dtype=torch.float32, device="cuda")
        qg.dequant(p, e, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), R.dequant_layer(layer, e))


def _dense(layer, acts, m, flags=0):
    p, buf = layers.prepare_layer(layer, compute_flags=flags)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    assert qg.workspace_bytes(p, m) == 0
    qg.gemm(p, x, xs, y, m, None)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(y)


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 33, 64, 65, 100, 300])
def test_dense_ragged_m(m):
    # 320 columns: a partial 128-column tile; K = 1280: ten 128-wide chunks over 4 or 8 waves
    layer, acts = synth.dense_w4a4_mxfp4(m=m, n=320, k=1280, seed=m)
    assert R.relative_error(_dense(layer, acts, m), R.dense_reference(layer, acts)) <= TOL


def test_dense_128_tiles_and_f16_output():
    # enough 128 x 128 tiles (16 x 32) for the large-M workgroup, a ragged last row tile
    m, n, k = 2000, 4096, 384
    layer, acts = synth.dense_w4a4_mxfp4(m=m, n=n, k=k, seed=3)
    assert R.relative_error(_dense(layer, acts, m), R.dense_reference(layer, acts)) <= TOL
    layer, acts = synth.dense_w4a4_mxfp4(m=40, n=192, k=256, out="f16", seed=4)
    assert R.relative_error(_dense(layer, acts, 40), R.dense_reference(layer, acts)) <= TOL


def test_dense_256_row_mfma_tiles():
    # enough 256 x 256 tiles (17 x 24) for the 256-row fp4 MFMA tiles, a ragged last row tile;
    # K = 512: two 256-wide steps
    m, n, k = 4100, 6144, 512
    layer, acts = synth.dense_w4a4_mxfp4(m=m, n=n, k=k, seed=21)
    assert R.relative_error(_dense(layer, acts, m), R.dense_reference(layer, acts)) <= TOL


def test_batch_invariant_rows_are_bitwise_equal():
    # one tile shape and no split over K for every M: a row's output does not depend on M
    layer, acts = synth.dense_w4a4_mxfp4(m=300, n=448, k=1024, seed=6)
    full = _dense(layer, acts, 300, qg.C_BATCH_INVARIANT)
    assert R.relative_error(full, R.dense_reference(layer, acts)) <= TOL
    for m in (1, 77):
        sub = synth.Acts(acts.x[:m], acts.x_scale[:m], None)
        assert np.array_equal(_dense(layer, sub, m, qg.C_BATCH_INVARIANT), full[:m])


def _moe(layer, acts, bm=None):
    t, topk = acts.topk_ids.shape
    p, buf = layers.prepare_layer(layer)
    bm = bm or qg.moe_block_m(p, t, topk)
    cs, cb = qg.moe_capacity(t, topk, layer.experts, bm)
    s = torch.empty(cs, dtype=torch.int32, device="cuda")
    e = torch.empty(cb, dtype=torch.int32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    ids = torch.from_numpy(np.ascontiguousarray(acts.topk_ids, np.int32)).cuda()
    qg.moe_align(ids, t, topk, layer.experts, bm, s, e, n)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((t * topk, layer.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert qg.workspace_bytes(p, t, topk) == 0
    qg.moe_gemm(p, x, xs, s, e, n, t, topk, bm, y, None)
    torch.cuda.synchronize()
    return bm, layers.out_bits_to_f64(y).reshape(t, topk, layer.n)


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_moe_every_block_size(bm):
    layer, acts = synth.moe_w4a4_mxfp4(t=90, experts=8, topk=3, n=320, k=640, seed=bm)
    acts.topk_ids[3, 1] = -1                                  # a dropped slot: not written
    _, y = _moe(layer, acts, bm)
    ref = R.moe_reference(layer, acts)
    assert np.all(np.isnan(y[3, 1]))
    ok = ~np.isnan(ref[:, :, 0])
    assert R.relative_error(y[ok], ref[ok]) <= TOL


@pytest.mark.parametrize("t", [1, 40, 700])
def test_moe_selected_block(t):
    layer, acts = synth.moe_w4a4_mxfp4(t=t, experts=8, topk=4, n=192, k=768, seed=t)
    bm, y = _moe(layer, acts)
    assert bm in (16, 32, 64, 128)
    assert R.relative_error(y, R.moe_reference(layer, acts)) <= TOL, f"block {bm}"


def test_moe_mfma_block_with_dropped_slot():
    # K = 768 (three 256-wide steps): 128-row blocks run on the MFMA kernel
    layer, acts = synth.moe_w4a4_mxfp4(t=300, experts=4, topk=2, n=320, k=768, seed=129)
    acts.topk_ids[5, 0] = -1
    _, y = _moe(layer, acts, 128)
    ref = R.moe_reference(layer, acts)
    assert np.all(np.isnan(y[5, 0]))
    ok = ~np.isnan(ref[:, :, 0])
    assert R.relative_error(y[ok], ref[ok]) <= TOL


def test_block_sizes_outside_the_kernel_are_rejected():
    layer, acts = synth.moe_w4a4_mxfp4(t=8, experts=4, topk=2, n=128, k=384, seed=2)
    with pytest.raises(qg.QGError):
        _moe(layer, acts, 4)
    with pytest.raises(qg.QGError):
        _moe(layer, acts, 256)


def test_dense_full_size_sampled():
    # N = 4096, K = 7168 (the MXFP4 workloads' shape) at M = 1, 64, 512 and 4096: sampled rows
    layer, acts = synth.dense_w4a4_mxfp4(m=4096, n=4096, k=7168, seed=0)
    cols = np.arange(0, layer.n, 37)
    w = R.dequant_rows(layer, 0, cols)
    for m in (1, 64, 512, 4096):
        sub = synth.Acts(acts.x[:m], acts.x_scale[:m], None)
        y = _dense(layer, sub, m)
        assert np.all(np.isfinite(y))
        rows = np.unique(np.concatenate([np.random.default_rng(m).choice(m, size=min(m, 8), replace=False), [m - 1]]))
        ref = R.dense_gemm(R.activations(synth.Acts(sub.x[rows], sub.x_scale[rows], None), "e2m1"), w)
        assert R.relative_error(y[np.ix_(rows, cols)], ref) <= TOL, f"M={m}"


# ---- MXFP4 activation quantizer -----------------------------------------------------------

def _quant_gpu(bits, in_type):
    rows, k = bits.shape
    x = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    codes = torch.full((rows, k // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, k // 32), 0xCD, dtype=torch.uint8, device="cuda")
    qg.quantize_e2m1_rows(x, rows, k, in_type, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _inputs(rows, k, seed, span, tiny):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)).astype(np.float32) * np.exp2(rng.integers(-span, span, size=(rows, 1)))
    x[0, :32] = 0.0                                                   # an all-zero block
    x[1, :32] = np.array([4.0, 2.5, -2.5, 0.25, 0.75, 1.25, 1.75, 3.5, 5.0, -5.0, 6.0, -0.0] + [0.5] * 20)  # ties
    x[1, 32:64] = 7.5 * np.sign(rng.standard_normal(32))            # saturation (amax < 8 * 2^E)
    x[2, 64:96] = np.arange(1, 33) * np.float32(tiny)                 # smallest magnitudes of the type
    return x


@pytest.mark.parametrize("in_type", ["bf16", "f16"])
def test_quantize_e2m1_rows_is_bit_exact(in_type):
    rows, k = 37, 4096
    if in_type == "bf16":
        bits = synth.f32_to_bf16_bits(_inputs(rows, k, 11, 30, 2.0 ** -130))
        vals, code = F.decode_bf16(bits), qg.A_BF16
    else:
        bits = synth.f32_to_f16_bits(_inputs(rows, k, 11, 8, 2.0 ** -20))
        vals, code = F.decode_f16(bits), qg.A_F16
    got_c, got_s = _quant_gpu(bits, code)
    ref_c, ref_s = Q.mxfp4_rows(vals)
    assert np.array_equal(got_s, ref_s)
    assert np.array_equal(got_c, ref_c)


def test_quantize_then_gemm_matches_the_oracle_chain():
    # bf16 activations -> MXFP4 on the GPU -> W4A4 product; the oracle quantizes the same values
    layer, _ = synth.dense_w4a4_mxfp4(m=1, n=256, k=1024, seed=12)
    m = 50
    bits = synth.f32_to_bf16_bits(np.random.default_rng(12).standard_normal((m, layer.k)).astype(np.float32))
    xq, xs = Q.mxfp4_rows(F.decode_bf16(bits))
    ref = R.dense_reference(layer, synth.Acts(xq, xs, None))
    x = torch.from_numpy(bits.view(np.int16)).cuda()
    codes = torch.empty((m, layer.k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((m, layer.k // 32), dtype=torch.uint8, device="cuda")
    qg.quantize_e2m1_rows(x, m, layer.k, qg.A_BF16, codes, scales)
    p, buf = layers.prepare_layer(layer)
    y = torch.empty((m, layer.n), dtype=torch.bfloat16, device="cuda")
    qg.gemm(p, codes, scales, y, m, None)
    torch.cuda.synchronize()
    assert R.relative_error(layers.out_bits_to_f64(y), ref) <= TOL
