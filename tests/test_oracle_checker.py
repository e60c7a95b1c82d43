"""Pins for the two oracle functions every GPU parity test leans on (CPU only).

* ``relative_error`` is the parity bar itself: max|Y - Y_ref| / max|Y_ref| over the whole
  tensor, non-finite GPU output counting as a failure.  A slip in it (a mean instead of a
  max, the GPU output in the denominator, a NaN that compares as a pass) would loosen every
  GPU test at once, so it is pinned by a hand-worked case and by properties that each
  plausible slip breaks; ``test_planted_checker_mistakes_fail_a_pin`` runs the same pins
  over such slips and requires each to fail one.
* ``dequant_rows`` (output channels picked out of one expert, used by the full-size checks
  on row subsets) must equal the corresponding rows of ``dequant_layer`` for every weight
  format, including block scales, where the scale row of channel n is n // block.
"""
import numpy as np
import pytest

from oracle import reference as R
from quantized_gemm_amd import synth


# ---- relative_error -------------------------------------------------------------------------

def _checker_pins(fn):
    """Each pin as (name, passed); a correct checker passes all of them."""
    out = []
    # hand-worked 2 x 2: |diff| = [[0.5, 0], [0, 0.25]], max|ref| = 4 -> 0.5 / 4 = 0.125
    ref = np.array([[1.0, -4.0], [2.0, 0.5]])
    got = np.array([[1.5, -4.0], [2.0, 0.25]])
    out.append(("2x2", fn(got, ref) == 0.125))
    # the max over elements, not the mean: one bad element among many good ones
    ref = np.ones((8, 8))
    got = ref.copy()
    got[3, 5] = 1.5
    out.append(("max not mean", fn(got, ref) == 0.5))
    # the denominator is max|Y_ref|, whatever the GPU output's magnitude
    ref = np.array([[2.0, -1.0]])
    got = np.array([[2.0, -9.0]])                 # |diff| 8, max|ref| 2, max|got| 9
    out.append(("denominator ref", fn(got, ref) == 4.0))
    # a negative reference element sets the denominator by its magnitude
    ref = np.array([[-8.0, 1.0]])
    got = np.array([[-8.0, 2.0]])
    out.append(("abs of ref", fn(got, ref) == 0.125))
    # identical tensors: exactly 0
    ref = np.arange(12.0).reshape(3, 4) - 5.0
    out.append(("equal", fn(ref.copy(), ref) == 0.0))
    # any non-finite GPU element is infinitely wrong, also where the reference is tiny
    for bad in (np.nan, np.inf, -np.inf):
        got = np.zeros((2, 3))
        got[1, 2] = bad
        v = fn(got, np.full((2, 3), 1e-3))
        out.append((f"non-finite {bad}", v == float("inf")))
    # errors in every direction count: a GPU value below the reference as much as above
    ref = np.array([[4.0, 4.0]])
    out.append(("sign", fn(np.array([[3.0, 4.0]]), ref) == fn(np.array([[5.0, 4.0]]), ref) == 0.25))
    # float32 / float16-valued inputs are compared in float64 (no overflow of the difference)
    ref = np.array([[60000.0, -60000.0]])
    got = np.array([[-60000.0, 60000.0]], dtype=np.float16)
    out.append(("float64 difference", fn(got, ref) == 2.0))
    return out


def test_relative_error_pins():
    failed = [name for name, ok in _checker_pins(R.relative_error) if not ok]
    assert not failed, failed


def _mean_checker(g, r):
    g = np.asarray(g, np.float64)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.mean(np.abs(g - r)) / np.max(np.abs(r)))


def _gpu_denominator(g, r):
    g = np.asarray(g, np.float64)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.max(np.abs(g - r)) / np.max(np.abs(g)))


def _nan_passes(g, r):
    # np.max propagates NaN and NaN <= tol is False, but nanmax quietly drops it
    g = np.asarray(g, np.float64)
    return float(np.nanmax(np.abs(g - r)) / np.max(np.abs(r)))


def _no_abs_denominator(g, r):
    g = np.asarray(g, np.float64)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.max(np.abs(g - r)) / np.max(r))


def _one_sided(g, r):
    g = np.asarray(g, np.float64)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(max(0.0, np.max(g - r)) / np.max(np.abs(r)))


def _native_precision(g, r):
    # difference taken in the GPU output's own type
    if not np.all(np.isfinite(np.asarray(g, np.float64))):
        return float("inf")
    d = np.abs(np.asarray(g) - np.asarray(r).astype(np.asarray(g).dtype)).astype(np.float64)
    return float(np.max(d) / np.max(np.abs(r)))


@pytest.mark.parametrize("mutant", [_mean_checker, _gpu_denominator, _nan_passes, _no_abs_denominator, _one_sided,
                                    _native_precision])
def test_planted_checker_mistakes_fail_a_pin(mutant):
    with np.errstate(all="ignore"):
        results = _checker_pins(mutant)
    assert any(not ok for _, ok in results), f"{mutant.__name__} passes every pin"


# ---- dequant_rows ---------------------------------------------------------------------------

def _layers():
    """One small layer of every weight format (several experts where the format has MoE use)."""
    out = {}
    out["int4 f16 group 128"] = synth.dense_w4a16_sym_f16(m=1, n=64, k=256, seed=1)[0]
    out["uint4 + zeros bf16 group 128"] = synth.dense_w4a16_asym_bf16(m=1, n=64, k=512, seed=2)[0]
    out["e4m3 per channel"] = synth.dense_w8a8_fp8(m=1, n=64, k=256, seed=3)[0]
    out["e4m3 128 x 128 blocks"] = synth.dense_w8a8_fp8_block(m=1, n=384, k=256, seed=4)[0]
    out["e4m3 blocks, MoE"] = synth.moe_w8a8_fp8_block(t=4, experts=3, topk=1, n=256, k=256, seed=5)[0]
    out["e2m1 UE8M0/32, MoE"] = synth.moe_w4a16_mxfp4(t=4, experts=3, topk=2, n=64, k=256, seed=6)[0]
    out["int4 -> e4m3 bf16 group 128, MoE"] = synth.moe_w4a8_int4(t=8, experts=4, topk=2, n=64, k=256, seed=7)[0]
    return out


def _rows_pins(fn):
    """For every format, expert and row set: fn(layer, e, rows) == dequant_layer(layer, e)[rows]."""
    bad = []
    rng = np.random.default_rng(0)
    for name, lay in _layers().items():
        for e in range(lay.experts):
            full = R.dequant_layer(lay, e)
            sets = [np.arange(lay.n), np.array([0]), np.array([lay.n - 1]),
                    np.unique(rng.choice(lay.n, size=9, replace=False)),
                    np.array([lay.n - 1, 3, 130 % lay.n, 129 % lay.n])]       # unsorted, across 128-row blocks
            for rows in sets:
                got = fn(lay, e, rows)
                if got.shape != (rows.size, lay.k) or not np.array_equal(got, full[rows]):
                    bad.append((name, e, rows.tolist()[:4]))
    return bad


def test_dequant_rows_equals_rows_of_the_full_dequantization():
    bad = _rows_pins(R.dequant_rows)
    assert not bad, bad[:5]


def test_block_scaled_layers_have_several_scale_rows():
    # the block-scaled layers above must span more than one 128-row scale block, or the
    # rows // block mapping would go unchecked
    lays = _layers()
    for name in ("e4m3 128 x 128 blocks", "e4m3 blocks, MoE"):
        lay = lays[name]
        assert lay.n // lay.group >= 2
        s = np.asarray(lay.s[0])
        assert not np.array_equal(s[0], s[1])


def _rows_scale_by_row(layer, expert, rows):
    # planted: block scales indexed by the row itself instead of its block
    rows = np.asarray(rows)
    s = np.asarray(layer.s[expert])
    if R.is_block_scaled(layer):
        srows = s[np.minimum(rows, s.shape[0] - 1)]
    else:
        srows = s[rows]
    z = None if layer.z is None else layer.z[expert][rows]
    return R.dequant_codes(layer.w[expert][rows], srows, z, layer.w_type, layer.s_type, layer.group, layer.k)


def _rows_zero_of_first_row(layer, expert, rows):
    # planted: zero points of the first selected row for every row
    rows = np.asarray(rows)
    z = None if layer.z is None else np.repeat(layer.z[expert][rows[:1]], rows.size, axis=0)
    return R.dequant_codes(layer.w[expert][rows], R._scale_rows(layer, expert, rows), z, layer.w_type, layer.s_type,
                           layer.group, layer.k)


def _rows_expert_zero(layer, expert, rows):
    # planted: the expert index ignored for the codes
    rows = np.asarray(rows)
    z = None if layer.z is None else layer.z[expert][rows]
    return R.dequant_codes(layer.w[0][rows], R._scale_rows(layer, expert, rows), z, layer.w_type, layer.s_type,
                           layer.group, layer.k)


def _rows_sorted(layer, expert, rows):
    # planted: rows returned in ascending order instead of the order asked for
    return R.dequant_rows(layer, expert, np.sort(np.asarray(rows)))


@pytest.mark.parametrize("mutant", [_rows_scale_by_row, _rows_zero_of_first_row, _rows_expert_zero, _rows_sorted])
def test_planted_row_subset_mistakes_fail_a_pin(mutant):
    assert _rows_pins(mutant), f"{mutant.__name__} passes every pin"
