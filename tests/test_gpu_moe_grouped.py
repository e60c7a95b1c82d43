"""GPU parity of the grouped MoE input organizations, through the C ABI.

qg_moe_grouped_map must equal the oracle's block map byte for byte (grouped-contiguous
offsets and grouped-masked counts, empty experts, counts outside [0, cap], many
workgroups); the grouped GEMM on those maps (qg_moe_gemm with tokens = rows_total,
topk = 1) must match the float64 reference y[r] = x[r] . W_e^T within the product bars,
and rows that belong to no expert must stay unwritten.
"""
import numpy as np
import pytest
import torch

import quantized_gemm_amd as qg
from quantized_gemm_amd import layers, synth
from oracle import align as A
from oracle import reference as R

pytestmark = pytest.mark.gpu

TOL16 = 5e-3
TOL8 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qg.lib()
    yield


def _map_gpu(layout, arr, experts, rows_total, cap, bm):
    cs, cb = qg.moe_capacity(rows_total, 1, experts, bm)
    s = torch.full((cs,), -7, dtype=torch.int32, device="cuda")
    e = torch.full((cb,), -7, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    a = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).cuda()
    qg.moe_grouped_map(qg.MOE_CONTIGUOUS if layout == "contiguous" else qg.MOE_MASKED, a, experts, rows_total, cap,
                       bm, s, e, n)
    torch.cuda.synchronize()
    return s, e, n


def _counts(rng, experts, mean, empty=2):
    c = rng.poisson(mean, size=experts)
    c[rng.choice(experts, size=min(empty, experts), replace=False)] = 0
    return c


@pytest.mark.parametrize("experts,mean,bm", [(1, 5, 4), (8, 20, 16), (128, 64, 64), (64, 700, 128), (1024, 3, 1),
                                             (16, 3000, 256)])
def test_contiguous_map_is_bit_exact(experts, mean, bm):
    rng = np.random.default_rng(experts + bm)
    offs = np.concatenate([[0], np.cumsum(_counts(rng, experts, mean))]).astype(np.int32)
    rows_total = int(offs[-1]) + 5                       # a few trailing rows outside every expert
    s, e, n = _map_gpu("contiguous", offs, experts, rows_total, 0, bm)
    rs, re_, rn = A.grouped_map("contiguous", offs, experts, bm, rows_total=rows_total)
    assert int(n.item()) == rn
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(e.cpu().numpy(), re_)


@pytest.mark.parametrize("experts,cap,bm", [(4, 8, 4), (32, 100, 16), (256, 40, 64), (8, 600, 128)])
def test_masked_map_is_bit_exact(experts, cap, bm):
    rng = np.random.default_rng(experts * cap)
    counts = rng.integers(-3, cap + 5, size=experts).astype(np.int32)     # clamped to [0, cap]
    counts[0] = 0
    s, e, n = _map_gpu("masked", counts, experts, experts * cap, cap, bm)
    rs, re_, rn = A.grouped_map("masked", counts, experts, bm, cap)
    assert int(n.item()) == rn
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(e.cpu().numpy(), re_)


def _gemm(layer, x_bits, x_scale, s, e, n, rows_total, bm):
    p, buf = layers.prepare_layer(layer)
    x = layers.to_dev(x_bits)
    xs = None if x_scale is None else torch.from_numpy(np.ascontiguousarray(x_scale)).cuda()
    y = torch.full((rows_total, layer.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(1, qg.workspace_bytes(p, rows_total, 1)), dtype=torch.uint8, device="cuda")
    qg.moe_gemm(p, x, xs, s, e, n, rows_total, 1, bm, y, ws)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(y)


def _ref(layer, x_bits, x_scale, row_experts):
    acts = synth.Acts(x_bits, x_scale, row_experts.reshape(-1, 1).astype(np.int32))
    return R.moe_reference(layer, acts)[:, 0, :]


@pytest.mark.parametrize("mean", [2, 30, 300])
def test_contiguous_gemm_mxfp4(mean):
    experts = 8
    rng = np.random.default_rng(mean)
    offs = np.concatenate([[0], np.cumsum(_counts(rng, experts, mean, empty=1))]).astype(np.int32)
    rows_total = int(offs[-1]) + 3
    layer, acts = synth.moe_w4a16_mxfp4(t=rows_total, experts=experts, topk=1, n=192, k=512, seed=mean)
    p, _ = layers.prepare_layer(layer)
    bm = qg.moe_block_m(p, int(offs[-1]), 1)
    s, e, n = _map_gpu("contiguous", offs, experts, rows_total, 0, bm)
    y = _gemm(layer, acts.x, None, s, e, n, rows_total, bm)
    ids = np.full(rows_total, -1)
    ids[:offs[-1]] = A.grouped_row_experts("contiguous", offs, experts)
    ref = _ref(layer, acts.x, None, ids)
    assert np.all(np.isnan(y[offs[-1]:]))                  # rows of no expert: not written
    ok = ids >= 0
    assert R.relative_error(y[ok], ref[ok]) <= TOL16, f"block {bm}"


@pytest.mark.parametrize("cap", [16, 200])
def test_masked_gemm_w4a8(cap):
    experts = 6
    rng = np.random.default_rng(cap)
    counts = rng.integers(0, cap + 1, size=experts).astype(np.int32)
    counts[2] = 0
    rows_total = experts * cap
    layer, acts = synth.moe_w4a8_int4(t=rows_total, experts=experts, topk=1, n=128, k=1024, seed=cap)
    p, _ = layers.prepare_layer(layer)
    bm = qg.moe_block_m(p, int(counts.sum()), 1)
    s, e, n = _map_gpu("masked", counts, experts, rows_total, cap, bm)
    y = _gemm(layer, acts.x, acts.x_scale, s, e, n, rows_total, bm)
    ids = A.grouped_row_experts("masked", counts, experts, cap)
    ref = _ref(layer, acts.x, acts.x_scale, ids)
    assert np.all(np.isnan(y[ids < 0]))
    ok = ids >= 0
    assert R.relative_error(y[ok], ref[ok]) <= TOL8, f"block {bm}"
