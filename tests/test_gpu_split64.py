"""GPU parity of the MFMA kernel's 64-row tiles with K split over workgroups, through the C ABI.

Few rows above the streaming sizes run as 64-row tiles with K split (up to 64 rows with 16-bit
activations, up to 128 with e4m3 activations), where the byte-operand loop issues five loads
over four MFMAs per step and the order of a slot's two loads carries the wait counts.  Each
case runs three times: the outputs must agree bit for bit (a stage read before it landed
would show as a run-to-run difference) and with the float64 oracle within the path's bar.
N = 2048 (8 column tiles) and K = 4096 so that the selector splits K (2 to 8 slices).
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


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qg.lib()
    yield


def _layer(kind, m):
    if kind == "e4m3":
        return synth.dense_w8a8_fp8(m=m, n=2048, k=4096, seed=m)
    if kind == "e4m3_block":
        return synth.dense_w8a8_fp8_block(m=m, n=2048, k=4096, seed=m)
    if kind == "w4a8_mxfp4":
        return synth.dense_w4a8_mxfp4(m=m, n=2048, k=4096, seed=m)
    return synth.dense_w4a16_asym_bf16(m=m, n=2048, k=4096, seed=m)


@pytest.mark.parametrize("kind,m", [("e4m3", 40), ("e4m3", 100), ("e4m3", 128), ("e4m3_block", 65),
                                    ("e4m3_block", 100), ("e4m3_block", 128), ("w4a8_mxfp4", 40),
                                    ("w4a8_mxfp4", 100), ("int4_bf16", 33), ("int4_bf16", 64)])
def test_split64_repeatable_and_exact(kind, m):
    layer, acts = _layer(kind, m)
    p, buf = layers.prepare_layer(layer)
    x, xs = layers.acts_to_dev(acts)
    ws_n = qg.workspace_bytes(p, m)
    assert ws_n > 0, "K should be split here"
    ws = torch.zeros(ws_n, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
        qg.gemm(p, x, xs, y, m, ws)
        torch.cuda.synchronize()
        outs.append(y.view(torch.int16).cpu().numpy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:]), "runs differ"
    got = layers.out_bits_to_f64(torch.from_numpy(outs[0]).view(layers.out_dtype(layer)))
    tol = TOL8 if layer.a_type == "e4m3" else TOL16
    assert R.relative_error(got, R.dense_reference(layer, acts)) <= tol
