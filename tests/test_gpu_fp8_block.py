"""GPU parity of block-scaled W8A8 (e4m3 weights with 128 x 128 block scales, e4m3
activations with one scale per (row, 128-wide K group)), through the C ABI.

Both kernel families: the streaming kernel up to 64 rows (and MoE blocks up to 64), the
block-scaled MFMA kernel above.  Bars: prepared bytes bit-exact; products
max|Y - Y_ref| / max|Y_ref| <= 2e-2 (e4m3 activations); with the batch-invariant flag, rows
bitwise independent of M.
"""
import numpy as np
import pytest
import torch

import quantized_gemm_amd as qg
from quantized_gemm_amd import layers, synth
from oracle import layout as L
from oracle import reference as R

pytestmark = pytest.mark.gpu

TOL8 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qg.lib()
    yield


def test_prepare_is_bit_exact():
    layer, _ = synth.moe_w8a8_fp8_block(t=2, experts=3, topk=1, n=256, k=384, seed=1)
    p, buf = layers.prepare_layer(layer)
    assert np.array_equal(buf.cpu().numpy(), L.repack(layer))


def _dense(layer, acts, m, flags=0):
    p, buf = layers.prepare_layer(layer, compute_flags=flags)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    ws = torch.zeros(max(1, qg.workspace_bytes(p, m)), dtype=torch.uint8, device="cuda")
    qg.gemm(p, x[:m], xs[:m], y, m, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("m,n,k", [(1, 384, 1152), (5, 384, 1152), (64, 512, 2048), (100, 512, 2048),
                                   (129, 384, 1152), (600, 768, 1024), (1, 1024, 4096)])
def test_dense(m, n, k):
    # 1..64 rows: the streaming kernel (4-row tiles; 16..64-row tiles with K split over
    # workgroups); above: the block-scaled MFMA kernel, split over K when its tiles are few
    layer, acts = synth.dense_w8a8_fp8_block(m=m, n=n, k=k, seed=m + n)
    y = layers.out_bits_to_f64(_dense(layer, acts, m))
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL8


def test_dense_f16_output():
    layer, acts = synth.dense_w8a8_fp8_block(m=70, n=256, k=512, seed=3)
    layer.out_type = "f16"
    y = layers.out_bits_to_f64(_dense(layer, acts, 70))
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL8


def test_batch_invariant_rows():
    layer, acts = synth.dense_w8a8_fp8_block(m=1000, n=512, k=1024, seed=4)
    ref = _dense(layer, acts, 1000, qg.C_BATCH_INVARIANT).view(torch.int16).cpu().numpy()
    for m in (1, 7, 128, 300):
        got = _dense(layer, acts, m, qg.C_BATCH_INVARIANT).view(torch.int16).cpu().numpy()
        assert np.array_equal(got, ref[:m]), f"M={m}"


@pytest.mark.parametrize("t", [1, 30, 60, 300, 1100])
def test_moe(t):
    layer, acts = synth.moe_w8a8_fp8_block(t=t, experts=4, topk=2, n=256, k=512, seed=t)
    p, buf = layers.prepare_layer(layer)
    bm = qg.moe_block_m(p, t, 2)
    # streaming blocks for few rows per expert, else 128-row MFMA blocks; 256 from a mean of
    # 512 rows per expert
    assert bm in (4, 16, 32, 64, 128, 256)
    assert (bm == 256) == (t == 1100)
    cs, cb = qg.moe_capacity(t, 2, 4, bm)
    s = torch.empty(cs, dtype=torch.int32, device="cuda")
    e = torch.empty(cb, dtype=torch.int32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    qg.moe_align(torch.from_numpy(np.ascontiguousarray(acts.topk_ids)).cuda(), t, 2, 4, bm, s, e, n)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((t * 2, layer.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    qg.moe_gemm(p, x, xs, s, e, n, t, 2, bm, y)
    torch.cuda.synchronize()
    got = layers.out_bits_to_f64(y).reshape(t, 2, layer.n)
    assert R.relative_error(got, R.moe_reference(layer, acts)) <= TOL8


@pytest.mark.parametrize("m", [1, 64, 512, 4096])
def test_dense_full_size_sampled(m):
    # the dense W8A8 workload's shape (N = K = 7168) with block scales
    layer, acts = synth.dense_w8a8_fp8_block(m=m, n=7168, k=7168, seed=0)
    y = _dense(layer, acts, m)
    assert bool(torch.isfinite(y).all())
    rng = np.random.default_rng(m)
    rows = np.unique(np.concatenate([rng.choice(m, size=min(m, 16), replace=False), [0, m - 1]]))
    cols = np.unique(np.concatenate([rng.choice(layer.n, size=48, replace=False), [0, layer.n - 1]]))
    got = layers.out_bits_to_f64(y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    sub = synth.Acts(acts.x[rows], acts.x_scale[rows], None)
    ref = R.dense_gemm(R.activations(sub, "e4m3"), R.dequant_rows(layer, 0, cols))
    assert R.relative_error(got, ref) <= TOL8
