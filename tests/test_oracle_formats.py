"""Pins for the oracle's value decoders (CPU only)."""
import numpy as np
import pytest
import torch

from conftest import load_golden
from oracle import formats as F
from quantized_gemm_amd import synth


def _vals(lst):
    return np.array([np.nan if v == "nan" else float(v) for v in lst])


def test_e2m1_table_matches_spec_fixture():
    g = load_golden("e2m1_values.json")
    got = F.decode_e2m1(np.array(g["codes"]))
    exp = _vals(g["values"])
    assert np.array_equal(got, exp)
    assert np.array_equal(np.signbit(got), np.signbit(exp))


def test_e2m1_magnitudes_are_sign_symmetric():
    c = np.arange(8)
    assert np.array_equal(F.decode_e2m1(c | 8), -F.decode_e2m1(c))


def test_e4m3_all_codes_match_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = F.decode_e4m3(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2  # only S.1111.111


def test_e4m3_fixture_points():
    g = load_golden("e4m3_points.json")
    got = F.decode_e4m3(np.array(g["codes"]))
    exp = _vals(g["values"])
    assert np.array_equal(np.isnan(got), np.isnan(exp))
    ok = ~np.isnan(exp)
    assert np.array_equal(got[ok], exp[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(exp[ok]))


def test_ue8m0_fixture_points():
    g = load_golden("ue8m0_points.json")
    got = F.decode_ue8m0(np.array(g["bytes"]))
    exp = _vals(g["values"])
    assert np.array_equal(np.isnan(got), np.isnan(exp))
    ok = ~np.isnan(exp)
    assert np.array_equal(got[ok], exp[ok])


def test_bf16_and_f16_decoders_match_library_casts():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4096) * 10.0 ** rng.integers(-6, 6, 4096)).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.decode_bf16(bits), ref)
    hb = synth.f32_to_f16_bits(np.clip(x, -60000, 60000))
    assert np.array_equal(F.decode_f16(hb), hb.view(np.float16).astype(np.float64))


def test_int4_decoders_and_int4_values_are_exact_e4m3_values():
    c = np.arange(16)
    assert np.array_equal(F.decode_int4(c, signed=False), np.arange(16.0))
    s = F.decode_int4(c, signed=True)
    assert sorted(s.tolist()) == list(range(-8, 8))
    assert s[8] == -8 and s[15] == -1 and s[7] == 7
    # Like the pages' statement that a zero-exponent float format holds exactly the symmetric
    # integers of its width: every int4 value is an exact e4m3 value, so the int4 -> e4m3
    # conversion the W4A8 path performs is lossless.
    e4 = F.decode_e4m3(np.arange(256))
    assert set(s.tolist()) <= set(e4[np.isfinite(e4)].tolist())


def test_nibble_unpack_roundtrip_iota_and_random():
    rng = np.random.default_rng(0)
    nib = rng.integers(0, 16, size=(5, 64))
    nib[0] = np.arange(64) % 16
    w = synth.pack_nibbles_u32(nib)
    assert np.array_equal(F.unpack_u32_nibbles(w), nib)
    b = synth.pack_nibbles_u8(nib)
    assert np.array_equal(F.unpack_u8_nibbles(b), nib)
    # element k sits at bits 4*(k%8): iota row word 0 must be 0x76543210
    assert w[0, 0] == 0x76543210
    assert b[0, 0] == 0x10 and b[0, 1] == 0x32
