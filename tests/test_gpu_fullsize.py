"""GPU parity at the workloads' full sizes, on sampled outputs.

Every launch here is the one the benchmark times: the same shapes, the same C-ABI calls
(qg_gemm with the workspace qg_workspace_bytes asks for; qg_moe_align + qg_moe_gemm with
the block size qg_moe_block_m picks), hence the same tile, split-K and kernel choice.
The full outputs are too large for the float64 oracle, so each launch is checked on a
seeded sample: output rows (dense) or (token, slot) pairs (MoE), always including the
first and last, times a seeded set of columns including the first and last.  The
oracle computes those elements one by one from the storage-form weights; the bar is the
same as for the small cases, max|Y - Y_ref| / max|Y_ref| over the sample, and every
output element must be finite.
"""
import numpy as np
import pytest
import torch

import quantized_gemm_amd as qg
from quantized_gemm_amd import layers, synth
from oracle import reference as R

pytestmark = pytest.mark.gpu

TOL16 = 5e-3
TOL8 = 2e-2
N_ROWS = 24
N_COLS = 48


def _tol(layer):
    return TOL8 if layer.a_type == "e4m3" else TOL16


def _sample(rng, total, count):
    pick = rng.choice(total, size=min(total, count), replace=False)
    return np.unique(np.concatenate([pick, [0, total - 1]]))


def _dense_check(layer, acts, m, seed):
    p, buf = layers.prepare_layer(layer)
    x, xs = layers.acts_to_dev(acts)
    x, xs = x[:m], (None if xs is None else xs[:m])
    y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    ws = torch.zeros(max(1, qg.workspace_bytes(p, m)), dtype=torch.uint8, device="cuda")
    qg.gemm(p, x, xs, y, m, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "non-finite output"
    rng = np.random.default_rng(seed)
    rows, cols = _sample(rng, m, N_ROWS), _sample(rng, layer.n, N_COLS)
    got = layers.out_bits_to_f64(y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    sub = synth.Acts(acts.x[rows], None if acts.x_scale is None else acts.x_scale[rows], None)
    ref = R.dense_gemm(R.activations(sub, layer.a_type), R.dequant_rows(layer, 0, cols))
    err = R.relative_error(got, ref)
    assert err <= _tol(layer), f"m={m}: relative error {err:.3g}"


@pytest.fixture(scope="module")
def c2():
    return synth.dense_w4a16_asym_bf16(m=4096, n=8192, k=8192, seed=0)


@pytest.mark.parametrize("m", [1, 16, 128, 1024, 4096])
def test_dense_w4a16_asym_bf16_8192(c2, m):
    layer, acts = c2
    _dense_check(layer, acts, m, seed=m)


@pytest.fixture(scope="module")
def c3():
    return synth.dense_w8a8_fp8(m=4096, n=7168, k=7168, seed=0)


@pytest.mark.parametrize("m", [1, 64, 512, 4096])
def test_dense_w8a8_fp8_7168(c3, m):
    layer, acts = c3
    _dense_check(layer, acts, m, seed=m)


def _moe_check(layer, acts, seed):
    t, topk = acts.topk_ids.shape
    p, buf = layers.prepare_layer(layer)
    bm = qg.moe_block_m(p, t, topk)
    cs, cb = qg.moe_capacity(t, topk, layer.experts, bm)
    ids = torch.from_numpy(np.ascontiguousarray(acts.topk_ids, dtype=np.int32)).cuda()
    sid = torch.empty(cs, dtype=torch.int32, device="cuda")
    eid = torch.empty(cb, dtype=torch.int32, device="cuda")
    npp = torch.empty(1, dtype=torch.int32, device="cuda")
    qg.moe_align(ids, t, topk, layer.experts, bm, sid, eid, npp)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((t * topk, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    ws = torch.zeros(max(1, qg.workspace_bytes(p, t, topk)), dtype=torch.uint8, device="cuda")
    qg.moe_gemm(p, x, xs, sid, eid, npp, t, topk, bm, y, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "non-finite output"
    rng = np.random.default_rng(seed)
    slots, cols = _sample(rng, t * topk, N_ROWS), _sample(rng, layer.n, N_COLS)
    got = layers.out_bits_to_f64(y[torch.from_numpy(slots).cuda()][:, torch.from_numpy(cols).cuda()])
    tok = slots // topk
    xa = R.activations(synth.Acts(acts.x[tok], None if acts.x_scale is None else acts.x_scale[tok], None),
                       layer.a_type)
    ref = np.empty_like(got)
    for i, sl in enumerate(slots):
        e = int(acts.topk_ids[sl // topk, sl % topk])
        ref[i] = R.dense_gemm(xa[i:i + 1], R.dequant_rows(layer, e, cols))[0]
    err = R.relative_error(got, ref)
    assert err <= _tol(layer), f"T={t}: relative error {err:.3g}"


@pytest.mark.parametrize("t", [16, 256, 4096])
def test_moe_w4a16_mxfp4_e128(t):
    layer, acts = synth.moe_w4a16_mxfp4(t=t, experts=128, topk=8, n=4096, k=7168, seed=0)
    _moe_check(layer, acts, seed=t)


@pytest.mark.parametrize("t", [64, 1024, 8192])
def test_moe_w4a8_int4_e64_skewed(t):
    layer, acts = synth.moe_w4a8_int4(t=t, experts=64, topk=6, n=2816, k=4096, seed=0)
    _moe_check(layer, acts, seed=t)
