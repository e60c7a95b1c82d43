"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bars: prepared bytes, read-back dequantization and MoE align are bit-exact;
GEMM outputs satisfy max|Y - Y_ref| / max|Y_ref| <= 5e-3 for f16/bf16 activations and
<= 2e-2 for e4m3 activations (Y_ref unrounded float64).
"""
import numpy as np
import pytest
import torch

import quantized_gemm_amd as qg
from quantized_gemm_amd import layers, synth
from oracle import align as A
from oracle import layout as L
from oracle import reference as R

pytestmark = pytest.mark.gpu

TOL16 = 5e-3
TOL8 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qg.lib()  # fail loudly if the HIP library is missing
    yield


def _tol(layer):
    return TOL8 if layer.a_type == "e4m3" else TOL16


SMALL = {
    "c1": lambda s: synth.dense_w4a16_sym_f16(m=16, n=512, k=1024, seed=s),
    "c2": lambda s: synth.dense_w4a16_asym_bf16(m=8, n=256, k=1024, seed=s),
    "c3": lambda s: synth.dense_w8a8_fp8(m=8, n=128, k=512, seed=s),
    "c4": lambda s: synth.moe_w4a16_mxfp4(t=8, experts=4, topk=2, n=128, k=512, seed=s),
    "c5": lambda s: synth.moe_w4a8_int4(t=8, experts=3, topk=2, n=128, k=512, seed=s),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_prepare_is_bit_exact(name):
    layer, _ = SMALL[name](1)
    p, buf = layers.prepare_layer(layer)
    ref = L.repack(layer)
    got = buf.cpu().numpy()
    assert got.size == ref.size
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"
    # deterministic: a second transform gives the same bytes
    p2, buf2 = layers.prepare_layer(layer)
    assert torch.equal(buf, buf2)


@pytest.mark.parametrize("name", list(SMALL))
def test_dequant_readback_is_bit_exact(name):
    layer, _ = SMALL[name](2)
    p, buf = layers.prepare_layer(layer)
    for e in range(layer.experts):
        out = torch.empty((layer.n, layer.k), dtype=torch.float32, device="cuda")
        qg.dequant(p, e, out)
        torch.cuda.synchronize()
        ref = R.dequant_layer(layer, e)
        if layer.w_type == "e4m3":
            ref = ref.astype(np.float32)    # one correctly rounded product
        assert np.array_equal(out.cpu().numpy().astype(np.float64), np.asarray(ref, dtype=np.float64)), f"expert {e}"


def _run_dense(layer, acts, m):
    p, buf = layers.prepare_layer(layer)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    ws_n = qg.workspace_bytes(p, m)
    ws = torch.zeros(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    qg.gemm(p, x, xs, y, m, ws)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(y)


@pytest.mark.parametrize("m", [16])
def test_dense_w4a16_sym_f16_full_size(m):
    layer, acts = synth.dense_w4a16_sym_f16(m=m, n=512, k=1024, seed=0)
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL16


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 15, 16, 17, 31, 33, 64, 100, 129])
def test_dense_w4a16_asym_bf16_ragged_m(m):
    layer, acts = synth.dense_w4a16_asym_bf16(m=m, n=320, k=1280, seed=3)
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL16


@pytest.mark.parametrize("m", [1, 5, 64, 100])
def test_dense_w8a8_fp8_ragged_m(m):
    layer, acts = synth.dense_w8a8_fp8(m=m, n=192, k=768, seed=4)
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL8


@pytest.mark.parametrize("k", [256, 512, 9216])
def test_dense_reduction_lengths(k):
    # K below one wave's chunk budget and K beyond 64 chunks (several rounds per wave)
    layer, acts = synth.dense_w4a16_asym_bf16(m=4, n=128, k=k, seed=5)
    y = _run_dense(layer, acts, 4)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL16


def test_dense_is_deterministic():
    layer, acts = synth.dense_w4a16_asym_bf16(m=16, n=256, k=1024, seed=6)
    p, buf = layers.prepare_layer(layer)
    x, _ = layers.acts_to_dev(acts)
    y1 = torch.empty((16, 256), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)
    ws = torch.zeros(max(1, qg.workspace_bytes(p, 16)), dtype=torch.uint8, device="cuda")
    qg.gemm(p, x, None, y1, 16, ws)
    qg.gemm(p, x, None, y2, 16, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ---- MoE ---------------------------------------------------------------------------------

def _align_gpu(ids_np, experts, bm):
    t, topk = ids_np.shape
    cs, cb = qg.moe_capacity(t, topk, experts, bm)
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    s = torch.full((cs,), -7, dtype=torch.int32, device="cuda")
    e = torch.full((cb,), -7, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    qg.moe_align(ids, t, topk, experts, bm, s, e, n)
    torch.cuda.synchronize()
    return s, e, n


ALIGN_CASES = [
    ("uniform", 64, 6, 64, 16), ("one_token", 1, 8, 128, 16), ("all_one_expert", 50, 1, 8, 16),
    ("big_block", 300, 8, 128, 64), ("skewed", 1024, 6, 64, 32), ("tiny_block", 33, 3, 5, 1),
    ("many", 8192, 6, 64, 64), ("invalid_ids", 40, 4, 16, 8),
    # several workgroups, each sorting its own range (2048 ids per workgroup): ragged
    # ranges with invalid ids near their edges, and the largest expert count
    ("ragged_invalid", 5001, 5, 100, 16), ("max_experts", 3000, 8, 512, 128),
]


@pytest.mark.parametrize("case", ALIGN_CASES, ids=lambda c: c[0])
def test_moe_align_is_bit_exact(case):
    name, t, topk, experts, bm = case
    rng = np.random.default_rng(t * 7 + topk)
    if name == "all_one_expert":
        ids = np.full((t, topk), 3, np.int32)
    elif name == "skewed":
        _, acts = synth.moe_w4a8_int4(t=t, experts=experts, topk=topk, n=64, k=256, seed=1)
        ids = acts.topk_ids
    else:
        ids = np.stack([rng.permutation(experts)[:topk] for _ in range(t)]).astype(np.int32)
    if name == "invalid_ids":
        ids[0, 0] = -1
        ids[5, 2] = experts
    if name == "ragged_invalid":
        flat = ids.reshape(-1)
        for f in (0, 2047, 2048, 4095, 10000, flat.size - 1):
            flat[f] = -1 if f % 2 else experts + 3
    s, e, n = _align_gpu(ids, experts, bm)
    rs, re_, rn = A.moe_align(ids, experts, bm)
    assert int(n.item()) == rn
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(e.cpu().numpy(), re_)


def _run_moe(layer, acts, workspace=False, bm=None):
    t, topk = acts.topk_ids.shape
    p, buf = layers.prepare_layer(layer)
    bm = bm or qg.moe_block_m(p, t, topk)
    s, e, n = _align_gpu(acts.topk_ids, layer.experts, bm)
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((t * topk, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    ws = None
    if workspace:
        ws = torch.zeros(max(1, qg.workspace_bytes(p, t, topk)), dtype=torch.uint8, device="cuda")
    qg.moe_gemm(p, x, xs, s, e, n, t, topk, bm, y, ws)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(y).reshape(t, topk, layer.n)


@pytest.mark.parametrize("t", [1, 5, 16, 40, 200])
def test_moe_w4a16_mxfp4(t):
    layer, acts = synth.moe_w4a16_mxfp4(t=t, experts=8, topk=4, n=192, k=768, seed=t)
    y = _run_moe(layer, acts)
    ref = R.moe_reference(layer, acts)
    assert R.relative_error(y, ref) <= TOL16


@pytest.mark.parametrize("t", [1, 7, 64, 300])
def test_moe_w4a8_int4_skewed(t):
    layer, acts = synth.moe_w4a8_int4(t=t, experts=8, topk=3, n=128, k=1024, seed=t)
    y = _run_moe(layer, acts)
    ref = R.moe_reference(layer, acts)
    assert R.relative_error(y, ref) <= TOL8


def test_moe_dropped_slots_are_not_written():
    layer, acts = synth.moe_w4a16_mxfp4(t=6, experts=4, topk=2, n=64, k=256, seed=9)
    acts.topk_ids[2, 1] = -1
    acts.topk_ids[4, 0] = 4
    y = _run_moe(layer, acts)
    assert np.all(np.isnan(y[2, 1])) and np.all(np.isnan(y[4, 0]))
    ref = R.moe_reference(layer, acts)
    ok = ~np.isnan(ref)
    assert np.max(np.abs(y[ok] - ref[ok])) / np.max(np.abs(ref[ok])) <= TOL16


# ---- the MFMA-bound path (row counts above the streaming bucket) ------------------------

@pytest.mark.parametrize("m", [65, 128, 257, 600])
def test_dense_w4a16_asym_bf16_mfma_path(m):
    layer, acts = synth.dense_w4a16_asym_bf16(m=m, n=320, k=1280, seed=7)   # 320: a partial 256-column tile
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL16


@pytest.mark.parametrize("m", [100, 513])
def test_dense_w4a16_sym_f16_mfma_path(m):
    layer, acts = synth.dense_w4a16_sym_f16(m=m, n=512, k=1024, seed=8)
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL16


@pytest.mark.parametrize("group,k,m", [(0, 1024, 16), (0, 1024, 300), (0, 4096, 100), (256, 1024, 300),
                                         (384, 1536, 5), (384, 1536, 300), (384, 3072, 100)])
def test_dense_scale_group_sizes(group, k, m):
    # per-channel scales and groups other than 128, including one that is not a power of
    # two, on the streaming kernel (5, 16 rows), the MFMA kernel and its split-K form
    # (100 rows: one row tile, two column tiles, K split over workgroups)
    layer, acts = synth.dense_w4a16_asym_bf16(m=m, n=512, k=k, group=group, seed=20 + group)
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL16
    layer, acts = synth.dense_w4a16_sym_f16(m=m, n=512, k=k, group=group, seed=21 + group)
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL16


@pytest.mark.parametrize("kind", ["w4a16", "w8a8"])
def test_dense_mfma_tile_256_rows(kind):
    # 25 row tiles (the last one ragged) x 16 column tiles: enough tiles for the 256-row
    # tile (and the XCD-aware remap of tile ids)
    m, n, k = 6200, 4096, 256
    if kind == "w4a16":
        layer, acts = synth.dense_w4a16_asym_bf16(m=m, n=n, k=k, seed=9)
    else:
        layer, acts = synth.dense_w8a8_fp8(m=m, n=n, k=k, seed=9)
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= _tol(layer)


@pytest.mark.parametrize("m", [65, 300])
def test_dense_w8a8_fp8_mfma_path(m):
    layer, acts = synth.dense_w8a8_fp8(m=m, n=320, k=768, seed=10)
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL8


@pytest.mark.parametrize("t,experts,bm", [(400, 4, None), (1100, 4, None), (1100, 4, 256)])
def test_moe_w4a16_mxfp4_mfma_path(t, experts, bm):
    # 200 and 550 rows per expert: 128-row blocks (e2m1 weights never take 256 by themselves),
    # and 256-row blocks when the caller asks for them
    layer, acts = synth.moe_w4a16_mxfp4(t=t, experts=experts, topk=2, n=320, k=512, seed=11)
    y = _run_moe(layer, acts, bm=bm)
    assert R.relative_error(y, R.moe_reference(layer, acts)) <= TOL16


@pytest.mark.parametrize("t,experts", [(5, 8), (40, 8), (400, 4), (1100, 4)])
def test_moe_w8a8_fp8(t, experts):
    # e4m3 weights per expert: streaming blocks (10 rows per expert), then MFMA blocks of
    # 128 (200 rows per expert) and 256 rows (550 rows per expert)
    layer, acts = synth.moe_w8a8_fp8(t=t, experts=experts, topk=2, n=320, k=512, seed=17)
    y = _run_moe(layer, acts)
    assert R.relative_error(y, R.moe_reference(layer, acts)) <= TOL8


@pytest.mark.parametrize("m", [8, 48, 100, 300])
def test_dense_w4a8_int4_to_fp8(m):
    # the W4A8 layer used densely (one expert): streaming path at 8 rows, fp8 MFMA with
    # per-group promotion above 32 rows (48 rows: 64-row tiles with K split)
    layer, acts = synth.moe_w4a8_int4(t=m, experts=1, topk=1, n=320, k=1024, seed=12)
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL8


@pytest.mark.parametrize("t", [200, 1000])
def test_moe_w4a8_int4_mfma_path(t):
    # 100 / 500 rows per expert (skewed router): blocks of 128 / 256 rows on the fp8 MFMA kernel
    layer, acts = synth.moe_w4a8_int4(t=t, experts=4, topk=2, n=256, k=512, seed=13)
    y = _run_moe(layer, acts)
    assert R.relative_error(y, R.moe_reference(layer, acts)) <= TOL8


# ---- split K (few output tiles: K is split over workgroups, partials summed in order) ----

@pytest.mark.parametrize("m,k", [(65, 4096), (128, 8192), (200, 2048)])
def test_dense_split_k(m, k):
    # 2 / 2 / 4 output tiles of 128 x 256: K split 8 / 8 / 4 ways
    layer, acts = synth.dense_w4a16_asym_bf16(m=m, n=512, k=k, seed=14)
    p, _ = layers.prepare_layer(layer)
    assert qg.workspace_bytes(p, m) > 0
    y = _run_dense(layer, acts, m)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL16


def test_dense_w8a8_fp8_split_k():
    layer, acts = synth.dense_w8a8_fp8(m=100, n=256, k=4096, seed=15)
    y = _run_dense(layer, acts, 100)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL8


def test_dense_split_k_is_deterministic_and_checks_workspace():
    layer, acts = synth.dense_w4a16_asym_bf16(m=96, n=256, k=2048, seed=16)
    p, buf = layers.prepare_layer(layer)
    x, _ = layers.acts_to_dev(acts)
    need = qg.workspace_bytes(p, 96)
    assert need == 4 * 96 * 256 * 4      # 32 K steps: 4 slices of 8
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y1 = torch.empty((96, 256), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)
    qg.gemm(p, x, None, y1, 96, ws)
    qg.gemm(p, x, None, y2, 96, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    with pytest.raises(qg.QGError):
        qg.gemm(p, x, None, y1, 96, ws[: need - 16])
    with pytest.raises(qg.QGError):
        qg.gemm(p, x, None, y1, 96, None)


# ---- W4A8 above the streaming sizes: int4 -> e4m3 in the MFMA kernel --------------------
# Each 128-wide K step is one scale group: two 32x32x64 fp8 MFMAs from zero, promoted by the
# group scale; 128- and 256-row tiles, and split K (partials summed with the per-token scale).

@pytest.mark.parametrize("m", [100, 300, 700])
def test_dense_w4a8_e4m3_mfma(m):
    layer, acts = synth.moe_w4a8_int4(t=m, experts=1, topk=1, n=320, k=1024, seed=17)
    p, buf = layers.prepare_layer(layer)
    assert qg.workspace_bytes(p, m) == 0          # 8 K steps: no split
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((m, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    qg.gemm(p, x, xs, y, m, None)
    torch.cuda.synchronize()
    assert R.relative_error(layers.out_bits_to_f64(y), R.dense_reference(layer, acts)) <= TOL8


def test_dense_w4a8_e4m3_mfma_split_k():
    # 2 x 2 output tiles of 128 x 256 and 32 K steps: K split 4 ways over workgroups
    layer, acts = synth.moe_w4a8_int4(t=200, experts=1, topk=1, n=512, k=4096, seed=20)
    p, buf = layers.prepare_layer(layer)
    need = qg.workspace_bytes(p, 200)
    assert need == 4 * 200 * 512 * 4
    x, xs = layers.acts_to_dev(acts)
    y = torch.full((200, 512), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    with pytest.raises(qg.QGError):
        qg.gemm(p, x, xs, y, 200, None)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    qg.gemm(p, x, xs, y, 200, ws)
    torch.cuda.synchronize()
    assert R.relative_error(layers.out_bits_to_f64(y), R.dense_reference(layer, acts)) <= TOL8


def test_dense_w4a8_e4m3_mfma_256_row_tiles():
    # 3100 rows x 8192 columns: 13 x 32 tiles of 256 x 256, over 1.5 workgroups per CU
    layer, acts = synth.moe_w4a8_int4(t=3100, experts=1, topk=1, n=8192, k=256, seed=21)
    y = _run_dense(layer, synth.Acts(acts.x, acts.x_scale, None), 3100)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL8


@pytest.mark.parametrize("t", [1200, 2100])
def test_moe_w4a8_int4_256_row_blocks(t):
    # 600 / 1050 rows per expert on average: 256-row blocks
    layer, acts = synth.moe_w4a8_int4(t=t, experts=4, topk=2, n=256, k=512, seed=18)
    p, _ = layers.prepare_layer(layer)
    assert qg.moe_block_m(p, t, 2) == 256
    assert qg.workspace_bytes(p, t, 2) == 0
    y = _run_moe(layer, acts)
    assert R.relative_error(y, R.moe_reference(layer, acts)) <= TOL8


def test_dense_streaming_split_needs_workspace():
    # 16 rows of a 2048-column layer: 16 column groups x 8 K slices of weight streaming
    layer, acts = synth.dense_w4a16_asym_bf16(m=16, n=2048, k=4096, seed=19)
    p, buf = layers.prepare_layer(layer)
    assert qg.workspace_bytes(p, 16) == 8 * 16 * 2048 * 4
    assert qg.workspace_bytes(p, 4) == 0
    x, _ = layers.acts_to_dev(acts)
    y = torch.empty((16, 2048), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qg.QGError):
        qg.gemm(p, x, None, y, 16, None)
    y = _run_dense(layer, acts, 16)
    assert R.relative_error(y, R.dense_reference(layer, acts)) <= TOL16


def test_dense_split_graph_replays():
    # A captured split-K call (16 rows: weight streaming over 8 K slices, then the slice
    # reduction) replayed with alternating activations, with eager work and synchronisations
    # between the replays; every replay must match the oracle.
    layer, acts_a = synth.dense_w4a16_asym_bf16(m=16, n=2048, k=4096, seed=23)
    acts_b = synth.dense_w4a16_asym_bf16(m=16, n=2048, k=4096, seed=24)[1]
    p, buf = layers.prepare_layer(layer)
    xa, _ = layers.acts_to_dev(acts_a)
    xb, _ = layers.acts_to_dev(acts_b)
    ref_a, ref_b = R.dense_reference(layer, acts_a), R.dense_reference(layer, acts_b)
    ws = torch.zeros(qg.workspace_bytes(p, 16), dtype=torch.uint8, device="cuda")
    xs = xa.clone()
    y = torch.empty((16, 2048), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qg.gemm(p, xs, None, y, 16, ws, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qg.gemm(p, xs, None, y, 16, ws, stream=s)
    torch.cuda.synchronize()
    for xi, ref in [(xb, ref_b), (xa, ref_a), (xb, ref_b), (xa, ref_a)]:
        xs.copy_(xi)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert R.relative_error(layers.out_bits_to_f64(y), ref) <= TOL16


@pytest.mark.parametrize("name", ["asym_g0_n320", "sym_g384", "fp8_block", "mxfp4_n192"])
def test_prepare_writes_every_byte_of_the_image(name):
    # regions whose sizes are not multiples of 256 bytes: the padding up to the next region
    # must be written (zeros) whatever the buffer held before
    layer = {
        "asym_g0_n320": lambda: synth.dense_w4a16_asym_bf16(m=1, n=320, k=384, group=0, seed=1)[0],
        "sym_g384": lambda: synth.dense_w4a16_sym_f16(m=1, n=192, k=1152, group=384, seed=2)[0],
        "fp8_block": lambda: synth.moe_w8a8_fp8_block(t=1, experts=3, topk=1, n=256, k=384, seed=3)[0],
        "mxfp4_n192": lambda: synth.moe_w4a16_mxfp4(t=1, experts=3, topk=1, n=192, k=128, seed=4)[0],
    }[name]()
    desc = layers.desc_for(layer)
    buf = torch.full((qg.prepared_bytes(desc),), 0xAB, dtype=torch.uint8, device="cuda")
    w, s = layers.to_dev(layer.w), layers.to_dev(layer.s)
    z = None if layer.z is None else layers.to_dev(layer.z)
    qg.prepare(desc, w, s, z, buf)
    torch.cuda.synchronize()
    ref = L.repack(layer)
    got = buf.cpu().numpy()
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} bytes differ"
