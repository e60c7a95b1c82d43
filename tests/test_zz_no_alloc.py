"""qg_gemm_noalloc against qg_gemm (GPU).

The no-allocation entry point runs the same kernels as qg_gemm with the library's own
per-GPU scratch array as the workspace, so on the same inputs its output must equal
qg_gemm's bit for bit; it is also checked against the float64 oracle at the 16-bit bar.
Each case makes two calls in a row, the second on a smaller input, so the second call
finds the first call's partial sums in the scratch array.
"""
import numpy as np
import pytest
import torch

import quantized_gemm_amd as qg
from quantized_gemm_amd import layers, synth
from oracle import reference as R

pytestmark = pytest.mark.gpu


def _run_pair(layer, acts, m, with_ws=True):
    p, buf = layers.prepare_layer(layer)
    x, xs = layers.acts_to_dev(acts)
    xm, xsm = x[:m], (None if xs is None else xs[:m])
    y_ref = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    nws = qg.workspace_bytes(p, m) if with_ws else 0
    ws = torch.zeros(max(1, nws), dtype=torch.uint8, device="cuda") if nws else None
    qg.gemm(p, xm, xsm, y_ref, m, ws)
    y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    qg.gemm_noalloc(p, xm, xsm, y, m)
    torch.cuda.synchronize()
    return p, buf, y, y_ref, nws


def _check(layer, acts, m, y, y_ref, tol):
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"m={m}: differs from qg_gemm"
    sub = synth.Acts(acts.x[:m], None if acts.x_scale is None else acts.x_scale[:m], None)
    ref = R.dense_gemm(R.activations(sub, layer.a_type), R.dequant_layer(layer, 0))
    err = R.relative_error(layers.out_bits_to_f64(y), ref)
    assert err <= tol, f"m={m}: relative error {err:.3g}"


def test_scratch_size_is_stated():
    assert qg.noalloc_scratch_bytes() == 32 << 20


@pytest.mark.parametrize("ms", [(128, 16), (16, 5), (64, 3)])
def test_noalloc_equals_gemm_two_calls(ms):
    # W4A16 uint4 + zeros, N = K = 8192: M = 128 splits K over 8 MFMA workgroups (32 MiB of
    # partials, the whole array), M = 16 / 5 / 64 split the streaming kernel, M = 3 needs none
    layer, acts = synth.dense_w4a16_asym_bf16(m=max(ms), n=8192, k=8192, seed=3)
    for m in ms:
        _, _, y, y_ref, nws = _run_pair(layer, acts, m)
        if m in (128, 16, 64):
            assert 0 < nws <= qg.noalloc_scratch_bytes()
        _check(layer, acts, m, y, y_ref, 5e-3)


def test_noalloc_w4a8_split_k_two_calls():
    # W4A8 (int4 -> e4m3 in the MFMA kernel): 4200 rows x 512 columns split K over 2
    # workgroups (17 MB of partials), then 200 rows split 4 ways (1.6 MB)
    layer, acts = synth.moe_w4a8_int4(t=4200, experts=1, topk=1, n=512, k=4096, seed=2)
    for m in (4200, 200):
        p, buf, y, y_ref, nws = _run_pair(layer, synth.Acts(acts.x, acts.x_scale, None), m)
        assert 0 < nws <= qg.noalloc_scratch_bytes()
        _check(layer, synth.Acts(acts.x, acts.x_scale, None), m, y, y_ref, 2e-2)


def test_noalloc_rejects_bad_arguments_before_launch():
    layer, acts = synth.dense_w4a16_asym_bf16(m=16, n=256, k=256, seed=1)
    p, buf = layers.prepare_layer(layer)
    x, _ = layers.acts_to_dev(acts)
    y = torch.empty((16, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qg.QGError):
        qg.gemm_noalloc(p, None, None, y, 16)
    bad = qg.Prepared.from_buffer_copy(p)
    bad.magic = 0
    with pytest.raises(qg.QGError):
        qg.gemm_noalloc(bad, x, None, y, 16)
    qg.gemm_noalloc(p, x, None, y, 0)     # M == 0: a no-op
