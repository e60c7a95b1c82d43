"""GPU parity of the MoE layer around the grouped products, through the C ABI.

Steps: qg_moe_swiglu (f16/bf16 output, or per-row e4m3 codes + scales), the down product
(qg_moe_gemm with one input row per slot: tokens = T*topk, topk = 1 on the gate/up
align output), qg_moe_combine, and the whole layer.  Also: reduction lengths that are a
multiple of 128 but not of 256 (the W4A8 down product's K = 1408), and W4A8 scale groups
other than 128.

Bars (derived from the arithmetic; the oracle is float64):
* SwiGLU, 16-bit output: |gpu - ref| <= u_out * |ref| + 2^-16 * |ref| + 2^-24, where u_out is
  the unit roundoff of the output type (2^-8 bf16, 2^-11 f16) and 2^-16 covers the float32
  sigmoid;
* SwiGLU -> e4m3: with exactly representable activations (gate 32, so silu(gate) = 32 in
  float32 and float64 alike) codes and scales are bit-exact; otherwise scales agree to 2^-20
  relative and every dequantized value is within half an e4m3 step of the float64 activation
  (plus the float32 noise above);
* combine: |gpu - ref| <= u_out * |ref| + topk * 2^-23 * sum_j |w y| + 2^-24;
* products and the whole layer: max|Y - Y_ref| / max|Y_ref| <= 5e-3 (16-bit activations) or
  2e-2 (e4m3 activations), as for every product.
"""
import numpy as np
import pytest
import torch

import quantized_gemm_amd as qg
from quantized_gemm_amd import layers, synth
from oracle import formats as F
from oracle import moe_layer as ML
from oracle import reference as R

pytestmark = pytest.mark.gpu

TOL16 = 5e-3
TOL8 = 2e-2
U_OUT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}   # unit roundoff: half an ulp, relative
T_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16}
Q_OUT = {"bf16": qg.O_BF16, "f16": qg.O_F16}
Q_ACT = {"bf16": qg.A_BF16, "f16": qg.A_F16}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qg.lib()
    yield


def _bits_to_f64(bits, dtype):
    return F.decode_act(bits, dtype)


def _dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


# ---- SwiGLU ----------------------------------------------------------------------------

@pytest.mark.parametrize("rows,inter,din,dout", [(1, 8, "bf16", "bf16"), (37, 200, "bf16", "bf16"),
                                                 (64, 1408, "bf16", "bf16"), (5, 2048, "f16", "f16"),
                                                 (9, 96, "bf16", "f16"), (3, 4096, "f16", "bf16")])
def test_swiglu_16bit(rows, inter, din, dout):
    gu = synth.gate_up_values(rows, inter, din, seed=rows + inter)
    out = torch.full((rows, inter), float("nan"), dtype=T_DTYPE[dout], device="cuda")
    qg.moe_swiglu(_dev16(gu), rows, inter, Q_OUT[din], Q_ACT[dout], out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = ML.swiglu(_bits_to_f64(gu, din))
    bound = (U_OUT[dout] + 2.0 ** -16) * np.abs(ref) + 2.0 ** -24
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))


def _swiglu_e4m3_gpu(gu, rows, inter, din):
    codes = torch.full((rows, inter), 0x7F, dtype=torch.uint8, device="cuda")
    scale = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    qg.moe_swiglu(_dev16(gu), rows, inter, Q_OUT[din], qg.A_FP8_E4M3, codes, scale)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scale.cpu().numpy()


@pytest.mark.parametrize("rows,inter", [(6, 64), (11, 1408), (3, 8192)])
def test_swiglu_e4m3_is_bit_exact_on_exact_activations(rows, inter):
    # gate = 32: sigmoid(32) rounds to 1 in float32 (and silu(32) to 32 from float64), so
    # act = 32 * up exactly on both sides; the quantizer's decisions must then agree bit for bit
    v = synth.gate_up_values(rows, inter, "bf16", seed=inter).copy()
    v[:, :inter] = 0x4200                                  # bf16 bits of 32.0
    v[1, inter:] = 0                                       # an all-zero activation row
    codes, scale = _swiglu_e4m3_gpu(v, rows, inter, "bf16")
    _, rc, rs = ML.swiglu_e4m3(_bits_to_f64(v, "bf16"))
    assert np.array_equal(scale.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(codes, rc), f"{np.count_nonzero(codes != rc)} codes differ"


def _swiglu_e2m1_gpu(gu, rows, inter, din):
    codes = torch.full((rows, inter // 2), 0xAB, dtype=torch.uint8, device="cuda")
    e8 = torch.full((rows, inter // 32), 0xCD, dtype=torch.uint8, device="cuda")
    qg.moe_swiglu(_dev16(gu), rows, inter, Q_OUT[din], qg.A_FP4_E2M1, codes, e8)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), e8.cpu().numpy()


@pytest.mark.parametrize("rows,inter,din", [(6, 64, "bf16"), (11, 1408, "bf16"), (3, 2048, "f16")])
def test_swiglu_e2m1_is_bit_exact_on_exact_activations(rows, inter, din):
    # gates in {0, 32, 64, 128}: silu(g) is g in float32 (sigmoid rounds to 1) and rounds to g
    # from float64, so act = g * up is exact on both sides and the bfloat16 rounding and the
    # MXFP4 decisions must agree bit for bit (an all-zero block included)
    rng = np.random.default_rng(inter + rows)
    v = synth.gate_up_values(rows, inter, din, seed=inter).copy()
    gates = np.array([0.0, 32.0, 64.0, 128.0], np.float32)[rng.integers(0, 4, size=(rows, inter))]
    v[:, :inter] = synth.f32_to_bf16_bits(gates) if din == "bf16" else synth.f32_to_f16_bits(gates)
    if din == "f16":
        # f16 up values have 11 significant bits: g * up could then sit exactly on a bfloat16
        # tie, which the exact float32 product rounds to even and float64 (silu(g) = g (1 - eps))
        # rounds down.  Up values with 8 significant bits keep g * up itself a bfloat16 value.
        up = F.decode_f16(v[:, inter:]).astype(np.float32)
        up = F.decode_bf16(synth.f32_to_bf16_bits(up)).astype(np.float32)
        v[:, inter:] = synth.f32_to_f16_bits(up)
    v[0, :32] = v[0, :32] * 0                               # gate 0 on a whole block: zeros
    codes, e8 = _swiglu_e2m1_gpu(v, rows, inter, din)
    rc, re8 = ML.swiglu_mxfp4(_bits_to_f64(v, din))
    assert np.array_equal(e8, re8)
    assert np.array_equal(codes, rc), f"{np.count_nonzero(codes != rc)} code bytes differ"


@pytest.mark.parametrize("rows,inter,din", [(40, 1408, "bf16"), (7, 2048, "f16")])
def test_swiglu_e2m1_equals_swiglu_then_quantizer(rows, inter, din):
    # the fused output is defined as the 16-bit SwiGLU rounded to bfloat16 and then the MXFP4
    # row quantizer: both routes on the GPU must give the same bytes (the values themselves are
    # checked against the oracle above and in the layer test)
    gu = synth.gate_up_values(rows, inter, din, seed=5 * rows + inter)
    codes, e8 = _swiglu_e2m1_gpu(gu, rows, inter, din)
    act = torch.empty((rows, inter), dtype=torch.bfloat16, device="cuda")
    qg.moe_swiglu(_dev16(gu), rows, inter, Q_OUT[din], qg.A_BF16, act)
    c2 = torch.empty((rows, inter // 2), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((rows, inter // 32), dtype=torch.uint8, device="cuda")
    qg.quantize_e2m1_rows(act, rows, inter, qg.A_BF16, c2, s2)
    torch.cuda.synchronize()
    assert np.array_equal(codes, c2.cpu().numpy()) and np.array_equal(e8, s2.cpu().numpy())


@pytest.mark.parametrize("rows,inter,din", [(40, 1408, "bf16"), (7, 2048, "f16"), (2, 8, "bf16")])
def test_swiglu_e4m3_general(rows, inter, din):
    gu = synth.gate_up_values(rows, inter, din, seed=3 * rows + inter)
    codes, scale = _swiglu_e4m3_gpu(gu, rows, inter, din)
    act, rc, rs = ML.swiglu_e4m3(_bits_to_f64(gu, din))
    np.testing.assert_allclose(scale, rs, rtol=2.0 ** -20, atol=0)
    vals = F.decode_e4m3(codes) * scale.astype(np.float64)[:, None]
    a = np.abs(act) / scale.astype(np.float64)[:, None]
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3))
    bound = (0.5 * step * (1 + 2.0 ** -10) + 2.0 ** -16 * a) * scale.astype(np.float64)[:, None]
    assert np.all(np.abs(vals - act) <= bound)
    assert np.mean(codes == rc) >= 0.99       # differences only where float32 noise meets a rounding tie


# ---- combine ---------------------------------------------------------------------------

@pytest.mark.parametrize("t,topk,n,dtype,drop", [(1, 1, 8, "bf16", 0.0), (37, 6, 1416, "bf16", 0.2),
                                                 (16, 8, 7168, "bf16", 0.0), (9, 3, 64, "f16", 0.5)])
def test_combine(t, topk, n, dtype, drop):
    y, w, ids = synth.slot_outputs(t, topk, n, experts=16, dtype=dtype, drop_frac=drop, seed=t + n)
    if t > 1:
        ids[1, :] = -1                                     # a token with no routed slot -> zeros
    yd = _dev16(y)
    flat = ids.reshape(-1)
    ydev = yd.clone()
    ydev.view(torch.int16)[torch.from_numpy(np.nonzero(flat < 0)[0]).cuda()] = 0x7FC0   # NaN rows: never read
    out = torch.full((t, n), float("nan"), dtype=T_DTYPE[dtype], device="cuda")
    qg.moe_combine(ydev, torch.from_numpy(w).cuda(), torch.from_numpy(ids).cuda(), t, topk, 16, n, Q_OUT[dtype], out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    yv = _bits_to_f64(y, dtype).reshape(t, topk, n)
    ref = ML.combine(yv, w, ids, 16)
    mag = ML.combine(np.abs(yv), np.abs(w), ids, 16)
    bound = U_OUT[dtype] * np.abs(ref) + topk * 2.0 ** -23 * mag + 2.0 ** -24
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))
    if t > 1:
        assert np.all(got[1] == 0)


# ---- the down product: one input row per slot -------------------------------------------

def _align(ids, experts, bm):
    t, topk = ids.shape
    cs, cb = qg.moe_capacity(t, topk, experts, bm)
    s = torch.empty((cs,), dtype=torch.int32, device="cuda")
    e = torch.empty((cb,), dtype=torch.int32, device="cuda")
    n = torch.empty((1,), dtype=torch.int32, device="cuda")
    qg.moe_align(torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(), t, topk, experts, bm, s, e, n)
    return s, e, n


def _down_gpu(down, act_bits, act_scale, ids, bm=None, workspace=True):
    t, topk = ids.shape
    rows = t * topk
    p, buf = layers.prepare_layer(down)
    if bm is None:
        bm = qg.moe_block_m(p, rows, 1)
    s, e, n = _align(ids, down.experts, bm)
    x = _dev16(act_bits) if act_bits.dtype == np.uint16 else torch.from_numpy(act_bits).cuda()
    xs = None if act_scale is None else torch.from_numpy(act_scale).cuda()
    y = torch.full((rows, down.n), float("nan"), dtype=layers.out_dtype(down), device="cuda")
    ws = None
    if workspace:
        ws = torch.zeros(max(1, qg.workspace_bytes(p, rows, 1)), dtype=torch.uint8, device="cuda")
    qg.moe_gemm(p, x, xs, s, e, n, rows, 1, bm, y, ws)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(y).reshape(t, topk, down.n)


@pytest.mark.parametrize("t,bm", [(3, None), (40, None), (40, 4), (40, 64), (300, 128)])
def test_down_product_mxfp4_slot_rows(t, bm):
    experts, topk, hidden, inter = 8, 4, 256, 384
    _, acts = synth.moe_w4a16_mxfp4(t=t, experts=experts, topk=topk, n=64, k=256, seed=t)
    down = synth.moe_down_mxfp4(experts=experts, n=hidden, k=inter, seed=t + 1)
    a_bits, _ = synth.act_rows(t * topk, inter, "bf16", seed=t + 2)
    y = _down_gpu(down, a_bits, None, acts.topk_ids, bm)
    ref = ML.down_reference(down, _bits_to_f64(a_bits, "bf16").reshape(t, topk, inter), acts.topk_ids)
    assert R.relative_error(y, ref) <= TOL16


@pytest.mark.parametrize("t,workspace", [(5, True), (120, True), (120, False)])
def test_down_product_w4a8_k1408(t, workspace):
    # the W4A8 workload's down product: K = 2816 / 2 = 1408 (a multiple of 128, not of 256)
    experts, topk, hidden, inter = 6, 3, 256, 1408
    _, acts = synth.moe_w4a8_int4(t=t, experts=experts, topk=topk, n=64, k=256, seed=t)
    down = synth.moe_down_w4a8(experts=experts, n=hidden, k=inter, seed=t + 1)
    codes, sx = synth.act_rows(t * topk, inter, "e4m3", seed=t + 2)
    y = _down_gpu(down, codes, sx, acts.topk_ids, workspace=workspace)
    act = F.decode_e4m3(codes).reshape(t, topk, inter)
    ref = ML.down_reference(down, act, acts.topk_ids, a_scale=sx.reshape(t, topk))
    assert R.relative_error(y, ref) <= TOL8


# ---- reduction lengths 128 * odd, W4A8 scale groups ---------------------------------------

def _dense(layer, acts, m, workspace=True):
    p, buf = layers.prepare_layer(layer)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    ws = None
    if workspace:
        ws = torch.zeros(max(1, qg.workspace_bytes(p, m)), dtype=torch.uint8, device="cuda")
    qg.gemm(p, x, xs, y, m, ws)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(y)


@pytest.mark.parametrize("k", [640, 1408])
@pytest.mark.parametrize("m", [1, 4, 16, 64, 200, 600])
def test_dense_k_odd_multiple_of_128(k, m):
    layer, acts = synth.dense_w4a16_asym_bf16(m=m, n=320, k=k, seed=k + m)
    assert R.relative_error(_dense(layer, acts, m), R.dense_reference(layer, acts)) <= TOL16
    layer, acts = synth.dense_w8a8_fp8(m=m, n=192, k=k, seed=k + m + 1)
    assert R.relative_error(_dense(layer, acts, m), R.dense_reference(layer, acts)) <= TOL8


def _dense_w4a8(m, k, group, seed):
    layer, acts = synth.moe_w4a8_int4(t=m, experts=1, topk=1, n=320, k=k, group=group, seed=seed)
    return layer, synth.Acts(acts.x, acts.x_scale, None)


@pytest.mark.parametrize("group,k", [(128, 1408), (256, 1024), (0, 1280), (384, 1536)])
@pytest.mark.parametrize("m,workspace", [(3, True), (40, True), (200, True), (200, False)])
def test_dense_w4a8_groups_and_routes(group, k, m, workspace):
    layer, acts = _dense_w4a8(m, k, group, seed=group + k + m)
    y = _dense(layer, acts, m, workspace)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL8


@pytest.mark.parametrize("group", [256, 0])
@pytest.mark.parametrize("workspace", [True, False])
def test_moe_w4a8_groups_mfma(group, workspace):
    layer, acts = synth.moe_w4a8_int4(t=400, experts=4, topk=2, n=128, k=1024, group=group, seed=group + 1)
    t, topk = acts.topk_ids.shape
    p, buf = layers.prepare_layer(layer)
    bm = qg.moe_block_m(p, t, topk)
    assert bm >= 128                                      # the MFMA kernels
    s, e, n = _align(acts.topk_ids, layer.experts, bm)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((t * topk, layer.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(1, qg.workspace_bytes(p, t, topk)), dtype=torch.uint8, device="cuda") if workspace else None
    qg.moe_gemm(p, x, xs, s, e, n, t, topk, bm, y, ws)
    torch.cuda.synchronize()
    got = layers.out_bits_to_f64(y).reshape(t, topk, layer.n)
    assert R.relative_error(got, R.moe_reference(layer, acts)) <= TOL8


# ---- the whole layer --------------------------------------------------------------------

def run_layer_mxfp4(up, down, acts):
    """align -> gate/up product -> SwiGLU -> down product (slot rows) -> combine, all on the GPU."""
    t, topk = acts.topk_ids.shape
    rows, inter = t * topk, down.k
    pu, bu = layers.prepare_layer(up)
    pd, bd = layers.prepare_layer(down)
    bm = qg.moe_block_m(pu, t, topk)
    assert qg.moe_block_m(pd, rows, 1) == bm
    ids = torch.from_numpy(np.ascontiguousarray(acts.topk_ids, np.int32)).cuda()
    s, e, n = _align(acts.topk_ids, up.experts, bm)
    x, _ = layers.acts_to_dev(acts)
    y1 = torch.empty((rows, 2 * inter), dtype=torch.bfloat16, device="cuda")
    qg.moe_gemm(pu, x, None, s, e, n, t, topk, bm, y1)
    act = torch.empty((rows, inter), dtype=torch.bfloat16, device="cuda")
    qg.moe_swiglu(y1, rows, inter, qg.O_BF16, qg.A_BF16, act)
    y2 = torch.empty((rows, down.n), dtype=torch.bfloat16, device="cuda")
    qg.moe_gemm(pd, act, None, s, e, n, rows, 1, bm, y2)
    out = torch.full((t, down.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    qg.moe_combine(y2, torch.from_numpy(acts.topk_weights).cuda(), ids, t, topk, up.experts, down.n, qg.O_BF16, out)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(out)


@pytest.mark.parametrize("t", [1, 33, 300])
def test_moe_layer_mxfp4(t):
    experts, topk, hidden, inter = 8, 2, 512, 256
    up, acts = synth.moe_w4a16_mxfp4(t=t, experts=experts, topk=topk, n=2 * inter, k=hidden, seed=t)
    down = synth.moe_down_mxfp4(experts=experts, n=hidden, k=inter, seed=t + 100)
    got = run_layer_mxfp4(up, down, acts)
    ref = ML.moe_layer_reference(up, down, acts, acts.topk_weights)
    assert R.relative_error(got, ref) <= TOL16


def run_layer_w4a4(up, down, acts):
    """W4A4: align -> gate/up (MXFP4 activations) -> SwiGLU with MXFP4 output -> down product
    (slot rows) -> combine, all on the GPU."""
    t, topk = acts.topk_ids.shape
    rows, inter = t * topk, down.k
    pu, bu = layers.prepare_layer(up)
    pd, bd = layers.prepare_layer(down)
    bm = qg.moe_block_m(pu, t, topk)
    assert qg.moe_block_m(pd, rows, 1) == bm
    ids = torch.from_numpy(np.ascontiguousarray(acts.topk_ids, np.int32)).cuda()
    s, e, n = _align(acts.topk_ids, up.experts, bm)
    x, xs = layers.acts_to_dev(acts)
    y1 = torch.empty((rows, 2 * inter), dtype=torch.bfloat16, device="cuda")
    qg.moe_gemm(pu, x, xs, s, e, n, t, topk, bm, y1)
    aq = torch.empty((rows, inter // 2), dtype=torch.uint8, device="cuda")
    asc = torch.empty((rows, inter // 32), dtype=torch.uint8, device="cuda")
    qg.moe_swiglu(y1, rows, inter, qg.O_BF16, qg.A_FP4_E2M1, aq, asc)   # SwiGLU -> bf16 -> MXFP4
    y2 = torch.empty((rows, down.n), dtype=torch.bfloat16, device="cuda")
    qg.moe_gemm(pd, aq, asc, s, e, n, rows, 1, bm, y2)
    out = torch.full((t, down.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    qg.moe_combine(y2, torch.from_numpy(acts.topk_weights).cuda(), ids, t, topk, up.experts, down.n, qg.O_BF16, out)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(out)


@pytest.mark.parametrize("t", [1, 33, 300])
def test_moe_layer_w4a4(t):
    # both sides quantize the SwiGLU output to MXFP4; the GPU's float32 SwiGLU (fast exp) can move
    # an element across an e2m1 midpoint, a one-step change of that element: the FP8 layers' bar
    experts, topk, hidden, inter = 8, 2, 512, 256
    up, acts = synth.moe_w4a4_mxfp4(t=t, experts=experts, topk=topk, n=2 * inter, k=hidden, seed=t)
    down = synth.moe_down_w4a4_mxfp4(experts=experts, n=hidden, k=inter, seed=t + 100)
    got = run_layer_w4a4(up, down, acts)
    ref = ML.moe_layer_reference_mxfp4(up, down, acts, acts.topk_weights)
    assert R.relative_error(got, ref) <= TOL8


# ---- per-token e4m3 quantization of 16-bit activations -------------------------------------

@pytest.mark.parametrize("rows,k,dtype", [(1, 8, "bf16"), (37, 1408, "bf16"), (5, 2048, "f16"), (9, 4096, "bf16"),
                                          (3, 7168, "bf16"), (4, 8192, "f16")])
def test_quantize_e4m3_rows_is_bit_exact(rows, k, dtype):
    # the inputs are exact in float32, and both sides take every decision in float32 with
    # correctly rounded divisions and round-to-nearest-even: codes and scales must agree bit for bit
    from oracle import quant as Q
    bits, _ = synth.act_rows(rows, k, dtype, sigma=3.0, seed=rows + k)
    bits = bits.copy()
    if rows > 2:
        bits[1] = 0                                         # an all-zero row: scale 1, codes 0
        bits[2, :4] = (synth.f32_to_bf16_bits if dtype == "bf16" else synth.f32_to_f16_bits)(
            np.array([1e4, -3e-3, 6e-5, -6e-5], np.float32))
    codes = torch.full((rows, k), 0x7F, dtype=torch.uint8, device="cuda")
    scale = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    qg.quantize_e4m3_rows(_dev16(bits), rows, k, Q_ACT[dtype], codes, scale)
    torch.cuda.synchronize()
    rc, rs = Q.absmax_rows(F.decode_act(bits, dtype).astype(np.float32))
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), rc), f"{np.count_nonzero(codes.cpu().numpy() != rc)} codes differ"
