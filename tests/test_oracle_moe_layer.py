"""Pins for the oracle's MoE layer steps: SwiGLU, per-row e4m3 quantization, combine, down
product and the whole layer (CPU only)."""
import numpy as np
import pytest
import scipy.special
import torch

from conftest import load_golden
from oracle import formats as F
from oracle import moe_layer as ML
from oracle import reference as R
from quantized_gemm_amd import synth


# ---- SwiGLU ----------------------------------------------------------------------------

def test_swiglu_hand_worked_fixture():
    g = load_golden("swiglu_tiny.json")
    row = np.array([g["gate_up_row"]])
    got = ML.swiglu(row)[0]
    np.testing.assert_allclose(got, np.array(g["act"]), rtol=1e-14, atol=0)


def test_silu_matches_library_routines():
    x = np.linspace(-60, 60, 4001)
    np.testing.assert_allclose(ML.silu(x), x * scipy.special.expit(x), rtol=1e-13, atol=1e-300)
    t = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(ML.silu(x), t, rtol=1e-13, atol=1e-300)


def test_silu_identities():
    x = np.linspace(-30, 30, 1201)
    # silu(-x) = -x * sigmoid(-x) = -x * (1 - sigmoid(x)) = silu(x) - x
    np.testing.assert_allclose(ML.silu(-x), ML.silu(x) - x, rtol=0, atol=1e-12)
    assert ML.silu(np.array([0.0]))[0] == 0.0
    big = np.array([800.0, -800.0])            # exp(-g) overflows / underflows
    assert ML.silu(big)[0] == 800.0 and ML.silu(big)[1] == 0.0


def test_swiglu_halves_are_not_interchangeable():
    # gate is the FIRST half: silu(g)*u differs from silu(u)*g for g != u
    row = np.array([[1.0, 2.0, 3.0, 4.0]])
    assert not np.allclose(ML.swiglu(row), ML.swiglu(row[:, ::-1].copy()))
    # up == 1 reduces to silu(gate); a large gate has sigmoid 1, so act = gate * up
    g = np.array([[-2.0, 0.5, 3.0, 1.0, 1.0, 1.0]])
    np.testing.assert_allclose(ML.swiglu(g)[0], ML.silu(g[0, :3]), rtol=1e-15)
    h = np.array([[700.0, 700.0, -1.5, 2.5]])
    np.testing.assert_array_equal(ML.swiglu(h)[0], [-1050.0, 1750.0])


def test_swiglu_e4m3_round_trip_and_absmax():
    rng = np.random.default_rng(3)
    gu = rng.standard_normal((5, 2 * 96)) * 4
    gu[3] = 0.0                                     # all-zero row -> scale 1, codes 0
    act, codes, scale = ML.swiglu_e4m3(gu)
    assert scale.dtype == np.float32 and scale[3] == 1.0 and np.all(codes[3] == 0)
    vals = F.decode_e4m3(codes) * scale.astype(np.float64)[:, None]
    for r in range(5):
        if r == 3:
            continue
        i = np.argmax(np.abs(act[r].astype(np.float32)))
        assert abs(F.decode_e4m3(codes[r, i])) == 448.0        # the absmax element maps to +-448
        # round to nearest: error at most half a step of e4m3 (relative 2^-4, or 2^-10 absolute
        # for subnormals) of the scaled value
        a = np.abs(act[r]) / scale[r]
        step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 3))
        assert np.all(np.abs(vals[r] - act[r]) <= (0.5 * step + 1e-6 * a) * scale[r])


# ---- combine ---------------------------------------------------------------------------

def test_combine_worked_example_skips_dropped_slots():
    y = np.array([[[1.0, 2.0], [np.nan, np.nan], [8.0, -16.0]]])
    w = np.array([[0.5, 0.25, 0.125]])
    ids = np.array([[2, -1, 0]])
    np.testing.assert_array_equal(ML.combine(y, w, ids, 4)[0], [1.5, -1.0])
    ids_out = np.array([[2, 4, 0]])                 # id == E is outside [0, E) as well
    np.testing.assert_array_equal(ML.combine(y, w, ids_out, 4)[0], [1.5, -1.0])


def test_combine_brute_force_and_special_cases():
    rng = np.random.default_rng(5)
    t, topk, n, e = 6, 3, 8, 5
    y = rng.standard_normal((t, topk, n))
    w = rng.random((t, topk))
    ids = rng.integers(-1, e + 1, size=(t, topk))
    ref = np.zeros((t, n))
    for i in range(t):
        for j in range(topk):
            if 0 <= ids[i, j] < e:
                for c in range(n):
                    ref[i, c] += w[i, j] * y[i, j, c]
    np.testing.assert_allclose(ML.combine(y, w, ids, e), ref, rtol=1e-14, atol=1e-14)
    one = np.zeros((t, 1), dtype=np.int64)
    np.testing.assert_array_equal(ML.combine(y[:, :1], np.ones((t, 1)), one, e), y[:, 0])
    np.testing.assert_array_equal(ML.combine(y, np.zeros((t, topk)), np.zeros((t, topk), int), e), 0.0)


# ---- down product and the whole layer --------------------------------------------------

def _tiny_pair(seed=0, t=5, experts=3, topk=2, hidden=256, inter=128):
    up, acts = synth.moe_w4a16_mxfp4(t=t, experts=experts, topk=topk, n=2 * inter, k=hidden, seed=seed)
    down = synth.moe_down_mxfp4(experts=experts, n=hidden, k=inter, seed=seed + 1)
    return up, down, acts


def test_down_reference_is_per_slot_dense_product():
    up, down, acts = _tiny_pair()
    rng = np.random.default_rng(1)
    t, topk = acts.topk_ids.shape
    act = rng.standard_normal((t, topk, down.k))
    y = ML.down_reference(down, act, acts.topk_ids)
    for i in range(t):
        for j in range(topk):
            w = R.dequant_layer(down, int(acts.topk_ids[i, j]))
            ref = np.array([sum(act[i, j, kk] * w[c, kk] for kk in range(down.k)) for c in range(down.n)])
            np.testing.assert_allclose(y[i, j], ref, rtol=1e-12, atol=1e-12)


def test_layer_reduces_to_dense_chain_for_one_expert():
    # E = 1, topk = 1, weight 1: out = swiglu(X W1^T) W2^T, written with explicit loops
    up, acts = synth.moe_w4a16_mxfp4(t=3, experts=1, topk=1, n=64, k=64, seed=7)
    down = synth.moe_down_mxfp4(experts=1, n=64, k=32, seed=8)
    acts.topk_weights = np.ones((3, 1), np.float32)
    x = R.activations(acts, "bf16")
    w1, w2 = R.dequant_layer(up, 0), R.dequant_layer(down, 0)
    ref = np.zeros((3, 64))
    for i in range(3):
        h = [sum(x[i, k] * w1[c, k] for k in range(64)) for c in range(64)]
        a = [h[c] / (1.0 + np.exp(-h[c])) * h[32 + c] for c in range(32)]
        for c in range(64):
            ref[i, c] = sum(a[k] * w2[c, k] for k in range(32))
    got = ML.moe_layer_reference(up, down, acts, acts.topk_weights)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_layer_is_linear_in_routing_weights_and_permutes_with_tokens():
    up, down, acts = _tiny_pair(seed=2)
    w = acts.topk_weights.astype(np.float64)
    base = ML.moe_layer_reference(up, down, acts, w)
    np.testing.assert_allclose(ML.moe_layer_reference(up, down, acts, 2 * w), 2 * base, rtol=1e-14, atol=1e-12)
    p = np.array([4, 2, 0, 3, 1])
    acts_p = synth.Acts(acts.x[p], None, acts.topk_ids[p], acts.topk_weights[p])
    np.testing.assert_allclose(ML.moe_layer_reference(up, down, acts_p, w[p]), base[p], rtol=1e-14, atol=1e-12)


def test_router_weights_are_softmax_probabilities_of_the_chosen_experts():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((7, 16)).astype(np.float32)
    ids = synth.topk_from_logits(logits, 4)
    w = synth.router_weights(logits, ids)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), axis=1), rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)          # slots in descending probability
