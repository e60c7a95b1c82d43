"""Pins for the prepared-layout reference and the synthetic FP8 inputs (CPU only)."""
import numpy as np
import pytest

from oracle import layout as L
from oracle import quant as Q
from oracle import formats as F
from quantized_gemm_amd import synth


def _iota_layer(w_type, a_type, s_type, n, k, group, experts, has_zero):
    g = 1 if group == 0 else k // group
    rng = np.random.default_rng(1)
    if w_type == "e4m3":
        w = (np.arange(experts * n * k) % 251).astype(np.uint8).reshape(experts, n, k)
    else:
        nib = (np.arange(experts * n * k) * 7 + np.arange(experts * n * k) // 13) % 16
        nib = nib.reshape(experts, n, k)
        w = synth.pack_nibbles_u8(nib) if w_type == "e2m1" else synth.pack_nibbles_u32(nib)
    if s_type == "f32":
        s = rng.uniform(0.1, 1, (experts, n, g)).astype(np.float32)
    elif s_type == "ue8m0":
        s = rng.integers(100, 140, (experts, n, g)).astype(np.uint8)
    else:
        s = rng.integers(0, 65536, (experts, n, g)).astype(np.uint16)
    z = rng.integers(0, 16, (experts, n, g)).astype(np.uint8) if has_zero else None
    return synth.Layer("t", w_type, a_type, s_type, "bf16", n, k, group, experts, w, s, z)


CASES = [("int4", "f16", "f16", 128, False), ("uint4", "bf16", "bf16", 128, True),
         ("e2m1", "bf16", "ue8m0", 32, False), ("e4m3", "e4m3", "f32", 0, False),
         ("int4", "e4m3", "bf16", 128, False)]


@pytest.mark.parametrize("w_type,a_type,s_type,group,has_zero", CASES)
def test_unpack_inverts_repack(w_type, a_type, s_type, group, has_zero):
    lay = _iota_layer(w_type, a_type, s_type, 48, 256, group, 3, has_zero)
    buf = L.repack(lay)
    assert buf.size == L.sizes(w_type, s_type, 48, 256, group, 3, has_zero)["total"]
    w, s, z = L.unpack(buf, w_type, a_type, s_type, 48, 256, group, 3, has_zero)
    assert np.array_equal(w, lay.w) and np.array_equal(s, lay.s)
    if has_zero:
        assert np.array_equal(z, lay.z)


def _single(w_type, a_type, n, k, row, col, val):
    nib = np.zeros((1, n, k), dtype=np.int64)
    nib[0, row, col] = val
    w = synth.pack_nibbles_u8(nib) if w_type == "e2m1" else synth.pack_nibbles_u32(nib)
    s = np.zeros((1, n, k // 32), np.uint16) if w_type != "e2m1" else np.zeros((1, n, k // 32), np.uint8)
    st = "ue8m0" if w_type == "e2m1" else "bf16"
    return synth.Layer("t", w_type, a_type, st, "bf16", n, k, 32, 1, w, s, None)


def test_hand_placed_nibbles():
    # uint4, "pair" order: element (n=0, k=1) -> unit 0, word 0, nibble position 4 -> byte 2 low nibble
    buf = L.repack(_single("uint4", "bf16", 16, 64, 0, 1, 5))
    assert buf[2] == 0x05 and np.count_nonzero(buf[:512]) == 1
    # element (n=3, k=42): unit (nb 0, ku 1, c 3) at 256 + 48; word j=1, i=2 -> position 1 -> byte 4 high nibble
    buf = L.repack(_single("uint4", "bf16", 16, 64, 3, 42, 9))
    assert buf[256 + 48 + 4] == 0x90 and np.count_nonzero(buf[:512]) == 1
    # "quad" order (int4 for e4m3): element (n=0, k=4) -> position 1 -> byte 0 high nibble
    buf = L.repack(_single("int4", "e4m3", 16, 64, 0, 4, 3))
    assert buf[0] == 0x30
    # "natural" e2m1: element (n=17, k=33): nb 1 (offset 2*256), ku 1, c 1 -> 512+256+16, word 0, pos 1
    buf = L.repack(_single("e2m1", "bf16", 32, 64, 17, 33, 0xB))
    assert buf[512 + 256 + 16] == 0xB0
    # int4 with 16-bit activations is biased by 8: zero codes become 8 everywhere
    buf = L.repack(_single("int4", "f16", 16, 32, 0, 0, 0))
    assert buf[0] == 0x88 and buf[15] == 0x88


def test_e4m3_byte_placement():
    n, k = 32, 64
    w = np.zeros((1, n, k), np.uint8)
    w[0, 17, 21] = 0x5A
    lay = synth.Layer("t", "e4m3", "e4m3", "f32", "bf16", n, k, 0, 1, w, np.ones((1, n, 1), np.float32), None)
    buf = L.repack(lay)
    # nb=1, ku=1, c=1, i=5 -> ((1*4)+1)*256 + 16 + 5
    assert buf[5 * 256 + 16 + 5] == 0x5A and np.count_nonzero(buf[:n * k]) == 1


def test_synthetic_fp8_inputs_are_nearest_even_e4m3_of_absmax_scaled_rows():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((16, 512), dtype=np.float32)
    codes, scale = synth.absmax_e4m3_rows(x)
    rcodes, rscale = Q.absmax_rows(x)
    assert np.array_equal(scale, rscale)
    assert np.array_equal(codes, rcodes)
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(F.decode_e4m3(codes[np.arange(16), am])) == 448.0)
    # dequantized values are within half an e4m3 ulp (relative 2^-4) of the input, or subnormal-close
    back = F.decode_e4m3(codes) * scale[:, None]
    err = np.abs(back - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) + 1e-30)


def test_block_scaled_layout_round_trip():
    layer, _ = synth.moe_w8a8_fp8_block(t=2, experts=2, topk=1, n=256, k=256, seed=3)
    buf = L.repack(layer)
    w, s, z = L.unpack(buf, layer.w_type, layer.a_type, layer.s_type, layer.n, layer.k, layer.group, layer.experts, False)
    assert np.array_equal(w, layer.w) and np.array_equal(s, layer.s) and z is None
    assert buf.size == L.sizes("e4m3", "f32", 256, 256, 128, 2, False)["total"]
