"""Pins for the oracle's W4A4 MXFP4 product and its MXFP4 activation quantizer (CPU only).

The product: every value 2^(E-127) * e2m1 is a short binary fraction, so products and small
sums are exact in float64 and the vectorised oracle must equal triple loops over the golden
e2m1 value table.  The quantizer (OCP MX v1.0 reading: shared exponent floor(log2 amax) - 2,
nearest e2m1 value with ties to the even code, saturation at 6) is pinned by hand-worked ties,
by a brute-force nearest-value search over the 8 magnitudes, by exact round trips of values
already on the grid, and by the scale's defining inequality 4 <= amax / 2^E < 8.
"""
import numpy as np
import pytest

from conftest import load_golden
from oracle import quant as Q
from oracle import reference as R
from quantized_gemm_amd import synth

_G = load_golden("e2m1_values.json")
_VAL = dict(zip(_G["codes"], _G["values"]))     # code -> value, from the format's table


def _nib(packed, k):
    return (int(packed[k // 2]) >> (4 * (k % 2))) & 0xF


def test_w4a4_brute_force_is_exact():
    layer, acts = synth.dense_w4a4_mxfp4(m=3, n=16, k=64, seed=7)
    y = R.dense_reference(layer, acts)
    ref = np.zeros((3, 16))
    for m in range(3):
        for n in range(16):
            for k in range(64):
                xv = _VAL[_nib(acts.x[m], k)] * 2.0 ** (int(acts.x_scale[m, k // 32]) - 127)
                wv = _VAL[_nib(layer.w[0, n], k)] * 2.0 ** (int(layer.s[0, n, k // 32]) - 127)
                ref[m, n] += xv * wv
    assert np.array_equal(y, ref)


def test_w4a4_moe_brute_force_is_exact():
    layer, acts = synth.moe_w4a4_mxfp4(t=5, experts=3, topk=2, n=16, k=64, seed=8)
    acts.topk_ids[1, 1] = -1                                      # a dropped slot stays NaN
    y = R.moe_reference(layer, acts)
    assert np.all(np.isnan(y[1, 1]))
    for t in range(5):
        for j in range(2):
            e = int(acts.topk_ids[t, j])
            if e < 0:
                continue
            for n in (0, 7, 15):
                ref = sum(_VAL[_nib(acts.x[t], k)] * 2.0 ** (int(acts.x_scale[t, k // 32]) - 127) *
                          _VAL[_nib(layer.w[e, n], k)] * 2.0 ** (int(layer.s[e, n, k // 32]) - 127) for k in range(64))
                assert y[t, j, n] == ref


def test_w4a4_scale_shift_moves_the_product_by_a_power_of_two():
    layer, acts = synth.dense_w4a4_mxfp4(m=2, n=32, k=128, seed=9)
    y0 = R.dense_reference(layer, acts)
    acts.x_scale = (acts.x_scale.astype(np.int64) + 3).astype(np.uint8)
    assert np.array_equal(R.dense_reference(layer, acts), y0 * 8.0)


@pytest.mark.parametrize("q,code", [(0.25, 0), (0.2500001, 1), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4),
                                    (3.5, 6), (5.0, 6), (5.0001, 7), (6.0, 7), (7.9, 7), (-0.25, 0), (-0.3, 9),
                                    (-5.0, 14), (-100.0, 15), (0.0, 0), (-0.0, 0)])
def test_round_to_e2m1_ties_and_saturation(q, code):
    assert int(Q.round_to_e2m1(np.array([q]))[0]) == code


def test_round_to_e2m1_is_the_nearest_value():
    rng = np.random.default_rng(3)
    q = np.concatenate([rng.uniform(-7, 7, 4000), np.arange(-28, 29) / 4.0])
    got = Q.round_to_e2m1(q)
    mags = [_VAL[c] for c in range(8)]
    for qi, c in zip(q, got):
        a = min(abs(qi), 6.0)
        d = [abs(a - v) for v in mags]
        best = min(d)
        cands = [i for i in range(8) if d[i] == best]
        want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        if qi < 0 and want != 0:
            want |= 8
        assert int(c) == want, qi


def test_mxfp4_rows_scale_and_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 256)) * np.exp2(rng.integers(-20, 20, size=(6, 1)))
    x[2, 32:64] = 0.0                                           # an all-zero block
    codes, e8 = Q.mxfp4_rows(x)
    assert codes.shape == (6, 128) and e8.shape == (6, 8)
    assert np.all(e8[2, 1] == 0) and np.all(codes[2, 16:32] == 0)
    for r in range(6):
        for b in range(8):
            blk = x[r, 32 * b:32 * b + 32]
            amax = np.max(np.abs(blk))
            if amax == 0:
                continue
            sc = 2.0 ** (int(e8[r, b]) - 127)
            assert 4.0 <= amax / sc < 8.0                       # E = floor(log2 amax) - 2
            dq = np.array([_VAL[_nib(codes[r], k)] for k in range(32 * b, 32 * b + 32)]) * sc
            q = np.abs(blk) / sc
            bound = np.where(q < 2, 0.25, np.where(q < 4, 0.5, np.where(q <= 6, 1.0, q - 6.0))) * sc
            assert np.all(np.abs(dq - blk) <= bound + 0.0)


def test_mxfp4_rows_round_trips_values_on_the_grid():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(4, 64))
    codes[:, 0] = 7                                             # each block reaches 6 * 2^E
    codes[:, 32] = 15
    e = rng.integers(-30, 30, size=(4, 2))
    x = np.array([[_VAL[int(c)] for c in row] for row in codes]) * np.exp2(np.repeat(e, 32, axis=1))
    got, e8 = Q.mxfp4_rows(x)
    canon = np.where(codes == 8, 0, codes)                      # -0 is written as +0
    assert np.array_equal(e8.astype(np.int64) - 127, e)
    unpacked = np.stack([got & 0xF, got >> 4], axis=-1).reshape(4, 64)
    assert np.array_equal(unpacked, canon)


def test_round_to_bf16_matches_the_cast_and_ties():
    import torch
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.standard_normal(5000) * np.exp2(rng.integers(-40, 40, 5000)),
                        np.exp2(-130.0) * np.arange(1, 50)])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().double().numpy()
    x32 = x.astype(np.float32).astype(np.float64)            # the cast rounds float32 inputs
    assert np.array_equal(Q.round_to_bf16(x32), ref)
    # hand ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 (-> 1, even); 1 + 3 * 2^-8 -> 1 + 2^-6
    assert Q.round_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert Q.round_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert Q.round_to_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)


def test_w4a4_layer_reference_brute_force():
    from oracle import moe_layer as ML
    up, acts = synth.moe_w4a4_mxfp4(t=3, experts=2, topk=2, n=64, k=64, seed=13)
    down = synth.moe_down_w4a4_mxfp4(experts=2, n=32, k=32, seed=14)
    acts.topk_ids[2, 1] = -1
    got = ML.moe_layer_reference_mxfp4(up, down, acts, acts.topk_weights)
    for t in range(3):
        out = np.zeros(32)
        for j in range(2):
            e = int(acts.topk_ids[t, j])
            if e < 0:
                continue
            y1 = [sum(_VAL[_nib(acts.x[t], k)] * 2.0 ** (int(acts.x_scale[t, k // 32]) - 127) *
                      _VAL[_nib(up.w[e, n], k)] * 2.0 ** (int(up.s[e, n, k // 32]) - 127) for k in range(64))
                  for n in range(64)]
            y1 = Q.round_to_bf16(np.array(y1))                     # the bf16 gate/up output
            act = [y1[i] / (1 + np.exp(-y1[i])) * y1[32 + i] for i in range(32)]
            codes, e8 = Q.mxfp4_rows(Q.round_to_bf16(np.array([act])))
            x2 = [_VAL[_nib(codes[0], k)] * 2.0 ** (int(e8[0, k // 32]) - 127) for k in range(32)]
            for n in range(32):
                out[n] += float(acts.topk_weights[t, j]) * sum(
                    x2[k] * _VAL[_nib(down.w[e, n], k)] * 2.0 ** (int(down.s[e, n, k // 32]) - 127) for k in range(32))
        assert np.allclose(got[t], out, rtol=1e-12, atol=1e-12 * np.max(np.abs(out)))
