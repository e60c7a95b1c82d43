"""GPU parity of W4A8 MXFP4 (e2m1 weights with UE8M0 block scales x per-token e4m3
activations), through the C ABI.

The product runs on the scaled fp8 x fp4 MFMAs of gfx950 with the weights as stored: the
streaming kernel (16x16x128) for up to 32 rows and MoE blocks up to 64, the MFMA kernel
(32x32x64) above, in 128- and 256-row tiles and split over K.  Bars: prepared bytes and
read-back bit-exact; products max|Y - Y_ref| / max|Y_ref| <= 2e-2 (e4m3 activations), and
much tighter in practice since the only rounding is the float32 accumulation and the
output conversion.
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


def test_prepare_and_readback_are_bit_exact():
    layer, _ = synth.moe_w4a8_mxfp4(t=4, experts=3, topk=2, n=128, k=512, seed=1)
    p, buf = layers.prepare_layer(layer)
    assert np.array_equal(buf.cpu().numpy(), L.repack(layer))
    for e in range(layer.experts):
        out = torch.empty((layer.n, layer.k), dtype=torch.float32, device="cuda")
        qg.dequant(p, e, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), R.dequant_layer(layer, e))


def _dense(layer, acts, m):
    p, buf = layers.prepare_layer(layer)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    ws = torch.zeros(max(1, qg.workspace_bytes(p, m)), dtype=torch.uint8, device="cuda")
    qg.gemm(p, x, xs, y, m, ws)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(y)


@pytest.mark.parametrize("m", [1, 3, 4, 5, 16, 33, 64, 65, 128, 300, 600])
def test_dense_ragged_m(m):
    # 320 columns: a partial 256-column tile; K = 1280: ten 128-wide steps
    layer, acts = synth.dense_w4a8_mxfp4(m=m, n=320, k=1280, seed=m)
    assert R.relative_error(_dense(layer, acts, m), R.dense_reference(layer, acts)) <= TOL8


@pytest.mark.parametrize("m,n,k", [(100, 512, 4096), (200, 1024, 2048)])
def test_dense_split_k(m, n, k):
    # few 128-row tiles: K split over workgroups, fp32 partials summed with the per-token scale
    layer, acts = synth.dense_w4a8_mxfp4(m=m, n=n, k=k, seed=m + 1)
    assert R.relative_error(_dense(layer, acts, m), R.dense_reference(layer, acts)) <= TOL8


def test_dense_256_row_tiles_and_f16_output():
    m, n, k = 6200, 4096, 256
    layer, acts = synth.dense_w4a8_mxfp4(m=m, n=n, k=k, seed=3)
    y = _dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL8
    layer, acts = synth.dense_w4a8_mxfp4(m=70, n=256, k=512, out="f16", seed=4)
    assert R.relative_error(_dense(layer, acts, 70), R.dense_reference(layer, acts)) <= TOL8


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
    ws = torch.zeros(max(1, qg.workspace_bytes(p, t, topk)), dtype=torch.uint8, device="cuda")
    qg.moe_gemm(p, x, xs, s, e, n, t, topk, bm, y, ws)
    torch.cuda.synchronize()
    return bm, layers.out_bits_to_f64(y).reshape(t, topk, layer.n)


@pytest.mark.parametrize("t,bm", [(1, None), (5, None), (40, None), (100, None), (300, None), (1100, None),
                                  (1100, 256)])
def test_moe(t, bm):
    # block sizes 4 and 16 (streaming), 128 (MFMA) as the routed rows per expert grow, and
    # 256-row MFMA blocks when the caller asks for them
    layer, acts = synth.moe_w4a8_mxfp4(t=t, experts=8, topk=4, n=192, k=768, seed=t)
    bm, y = _moe(layer, acts, bm)
    assert R.relative_error(y, R.moe_reference(layer, acts)) <= TOL8, f"block {bm}"


def test_moe_full_size_sampled():
    # the MXFP4 MoE workload's shapes (E=128 top-8, N=4096, K=7168) with e4m3 activations
    layer, acts = synth.moe_w4a8_mxfp4(t=4096, experts=128, topk=8, n=4096, k=7168, seed=0)
    for t in (16, 4096):
        sub = synth.Acts(acts.x[:t], acts.x_scale[:t], acts.topk_ids[:t], None)
        bm, y = _moe(layer, sub)
        assert np.all(np.isfinite(y))
        rng = np.random.default_rng(t)
        toks = np.unique(np.concatenate([rng.choice(t, size=min(t, 6), replace=False), [0, t - 1]]))
        cols = np.unique(np.concatenate([rng.choice(layer.n, size=48, replace=False), [0, layer.n - 1]]))
        xa = R.activations(synth.Acts(sub.x[toks], sub.x_scale[toks], None), "e4m3")
        got, ref = [], []
        for i, tk in enumerate(toks):
            for j in range(8):
                e = int(sub.topk_ids[tk, j])
                ref.append(R.dense_gemm(xa[i:i + 1], R.dequant_rows(layer, e, cols))[0])
                got.append(y[tk, j, cols])
        err = R.relative_error(np.array(got), np.array(ref))
        assert err <= TOL8, f"T={t} block {bm}: {err:.3g}"
