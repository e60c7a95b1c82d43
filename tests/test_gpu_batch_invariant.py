"""Batch-invariant execution (compute flag QG_C_BATCH_INVARIANT), through the C ABI.

With the flag every row count runs the same MFMA kernel without a split over K, so each
output row must be bitwise identical whatever the number of rows around it: the rows of
runs with M = 1 .. 1000 must equal the first rows of one large run.  The large run is also
checked against the oracle on a sample.
"""
import numpy as np
import pytest
import torch

import quantized_gemm_amd as qg
from quantized_gemm_amd import layers, synth
from oracle import reference as R

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qg.lib()
    yield


def _dense_rows(p, layer, x, xs, m, workspace=True):
    y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    ws = None
    if workspace:
        ws = torch.zeros(max(1, qg.workspace_bytes(p, m)), dtype=torch.uint8, device="cuda")
    qg.gemm(p, x[:m], None if xs is None else xs[:m], y, m, ws)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy()


CASES = {
    "w4a16_uint4": lambda m: synth.dense_w4a16_asym_bf16(m=m, n=8192, k=1024, seed=11),   # 256-row tiles at 4096
    "w8a8": lambda m: synth.dense_w8a8_fp8(m=m, n=1024, k=1024, seed=12),
    "w4a8_mxfp4": lambda m: synth.dense_w4a8_mxfp4(m=m, n=1024, k=1024, seed=13),
    "w4a8_int4": lambda m: (lambda la: (la[0], synth.Acts(la[1].x, la[1].x_scale, None)))(
        synth.moe_w4a8_int4(t=m, experts=1, topk=1, n=1024, k=1024, seed=14)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_dense_rows_do_not_depend_on_m(name):
    big = 4096
    layer, acts = CASES[name](big)
    p, buf = layers.prepare_layer(layer, compute_flags=qg.C_BATCH_INVARIANT)
    x, xs = layers.acts_to_dev(acts)
    ref = _dense_rows(p, layer, x, xs, big)
    for m in (1, 5, 16, 64, 65, 300, 1000):
        got = _dense_rows(p, layer, x, xs, m)
        assert np.array_equal(got, ref[:m]), f"M={m}: {np.count_nonzero(got != ref[:m])} elements differ"
    # the large run against the oracle on a sample of rows and columns
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(big, 8, replace=False), [0, big - 1]]))
    cols = np.unique(np.concatenate([rng.choice(layer.n, 32, replace=False), [0, layer.n - 1]]))
    sub = synth.Acts(acts.x[rows], None if acts.x_scale is None else acts.x_scale[rows], None)
    yref = R.dense_gemm(R.activations(sub, layer.a_type), R.dequant_rows(layer, 0, cols))
    got = torch.from_numpy(ref[rows][:, cols].copy()).view(layers.out_dtype(layer)).float().numpy()
    assert R.relative_error(got.astype(np.float64), yref) <= (2e-2 if layer.a_type == "e4m3" else 5e-3)


def test_moe_rows_do_not_depend_on_t():
    big = 600
    layer, acts = synth.moe_w4a16_mxfp4(t=big, experts=8, topk=2, n=256, k=512, seed=15)
    p, buf = layers.prepare_layer(layer, compute_flags=qg.C_BATCH_INVARIANT)
    x, _ = layers.acts_to_dev(acts)

    def run(t):
        bm = qg.moe_block_m(p, t, 2)
        assert bm >= 128
        cs, cb = qg.moe_capacity(t, 2, 8, bm)
        s = torch.empty(cs, dtype=torch.int32, device="cuda")
        e = torch.empty(cb, dtype=torch.int32, device="cuda")
        n = torch.empty(1, dtype=torch.int32, device="cuda")
        ids = torch.from_numpy(np.ascontiguousarray(acts.topk_ids[:t])).cuda()
        qg.moe_align(ids, t, 2, 8, bm, s, e, n)
        y = torch.full((t * 2, layer.n), float("nan"), dtype=torch.bfloat16, device="cuda")
        qg.moe_gemm(p, x[:t], None, s, e, n, t, 2, bm, y)
        torch.cuda.synchronize()
        return y.view(torch.int16).cpu().numpy()

    ref = run(big)
    for t in (1, 3, 40):
        assert np.array_equal(run(t), ref[:2 * t]), f"T={t}"
    # a streaming block size is refused under the flag
    cs, cb = qg.moe_capacity(4, 2, 8, 16)
    s = torch.empty(cs, dtype=torch.int32, device="cuda")
    e = torch.empty(cb, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.empty((8, layer.n), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qg.QGError):
        qg.moe_gemm(p, x[:4], None, s, e, n, 4, 2, 16, y)
