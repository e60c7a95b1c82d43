"""GPU parity at the workloads' full sizes, over whole output tensors.

Every launch here is the one the benchmark times: the same shapes, the same C-ABI calls
(qg_gemm with the workspace qg_workspace_bytes asks for; qg_moe_align + qg_moe_gemm with
the block size qg_moe_block_m picks), hence the same tile, split-K and kernel choice; MoE
sweeps take the first T tokens of one draw at the largest T, as the benchmark does.  The
whole output is compared element by element with the float64 oracle: dense outputs against
X . dequant(W)^T, MoE outputs expert by expert (each expert dequantized once and multiplied
with every (token, slot) row routed to it, over a thread pool).  The bar is the one of the
small cases, max|Y - Y_ref| / max|Y_ref| over the whole tensor, with any non-finite output
element a failure (outputs start as NaN, so an unwritten element fails too).

The MoE layers at the end of the file check sampled tokens (their oracle needs every gate/up
row of a token).
"""
import os
from concurrent.futures import ThreadPoolExecutor

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
POOL = max(1, min(8, (os.cpu_count() or 4) // 2))


def _tol(layer):
    return TOL8 if layer.a_type == "e4m3" else TOL16


def _sample(rng, total, count):
    pick = rng.choice(total, size=min(total, count), replace=False)
    return np.unique(np.concatenate([pick, [0, total - 1]]))


# ---- dense ----------------------------------------------------------------------------------

class _Dense:
    """One full-size dense layer on the GPU and its float64 dequantized weights."""

    def __init__(self, layer, acts):
        self.layer, self.acts = layer, acts
        self.p, self.buf = layers.prepare_layer(layer)
        self.x, self.xs = layers.acts_to_dev(acts)
        self.w_ref = R.dequant_layer(layer, 0)
        self.x_ref = R.activations(acts, layer.a_type)

    def check(self, m):
        lay = self.layer
        y = torch.full((m, lay.n), float("nan"), dtype=layers.out_dtype(lay), device="cuda")
        ws = torch.zeros(max(1, qg.workspace_bytes(self.p, m)), dtype=torch.uint8, device="cuda")
        qg.gemm(self.p, self.x[:m], None if self.xs is None else self.xs[:m], y, m, ws)
        torch.cuda.synchronize()
        got = layers.out_bits_to_f64(y)
        ref = R.dense_gemm(self.x_ref[:m], self.w_ref)
        err = R.relative_error(got, ref)
        assert err <= _tol(lay), f"m={m}: relative error {err:.3g} over the whole {m} x {lay.n} output"


@pytest.fixture(scope="module")
def c2():
    d = _Dense(*synth.dense_w4a16_asym_bf16(m=4096, n=8192, k=8192, seed=0))
    yield d
    del d


@pytest.mark.timeout(300)
@pytest.mark.parametrize("m", [1, 16, 128, 1024, 4096])
def test_dense_w4a16_asym_bf16_8192(c2, m):
    c2.check(m)


@pytest.fixture(scope="module")
def c3():
    d = _Dense(*synth.dense_w8a8_fp8(m=4096, n=7168, k=7168, seed=0))
    yield d
    del d


@pytest.mark.timeout(300)
@pytest.mark.parametrize("m", [1, 64, 512, 4096])
def test_dense_w8a8_fp8_7168(c3, m):
    c3.check(m)


@pytest.fixture(scope="module")
def c3_block():
    d = _Dense(*synth.dense_w8a8_fp8_block(m=4096, n=7168, k=7168, seed=0))
    yield d
    del d


@pytest.mark.timeout(300)
@pytest.mark.parametrize("m", [1, 64, 512, 4096])
def test_dense_w8a8_fp8_block_7168(c3_block, m):
    # 1 / 64 rows: streaming kernel; 512: 128-row tiles with K split; 4096: 256-row tiles
    c3_block.check(m)


def test_dense_w4a16_sym_f16_512x1024():
    d = _Dense(*synth.dense_w4a16_sym_f16(m=16, n=512, k=1024, seed=0))
    d.check(16)


# ---- MoE ------------------------------------------------------------------------------------

def _moe_gpu(p, layer, acts, t, with_ws=True):
    """One MoE launch on the first t tokens, as the benchmark makes it; output [t * topk, N] float64."""
    topk = acts.topk_ids.shape[1]
    bm = qg.moe_block_m(p, t, topk)
    cs, cb = qg.moe_capacity(t, topk, layer.experts, bm)
    ids = torch.from_numpy(np.ascontiguousarray(acts.topk_ids[:t], dtype=np.int32)).cuda()
    sid = torch.empty(cs, dtype=torch.int32, device="cuda")
    eid = torch.empty(cb, dtype=torch.int32, device="cuda")
    npp = torch.empty(1, dtype=torch.int32, device="cuda")
    qg.moe_align(ids, t, topk, layer.experts, bm, sid, eid, npp)
    x, xs = layers.acts_to_dev(acts)
    x, xs = x[:t], (None if xs is None else xs[:t])
    y = torch.full((t * topk, layer.n), float("nan"), dtype=layers.out_dtype(layer), device="cuda")
    nws = qg.workspace_bytes(p, t, topk) if with_ws else 0
    ws = torch.zeros(max(1, nws), dtype=torch.uint8, device="cuda") if nws else None
    qg.moe_gemm(p, x, xs, sid, eid, npp, t, topk, bm, y, ws)
    torch.cuda.synchronize()
    return layers.out_bits_to_f64(y)


def _moe_reference(layer, acts, ts):
    """Oracle outputs [t * topk, N] for every t in ts (first t tokens), one expert at a time."""
    ids = np.asarray(acts.topk_ids)
    topk = ids.shape[1]
    x = R.activations(acts, layer.a_type)
    refs = {t: np.full((t * topk, layer.n), np.nan) for t in ts}
    tmax = max(ts)
    used = np.unique(ids[:tmax][(ids[:tmax] >= 0) & (ids[:tmax] < layer.experts)])

    def one(e):
        tt, jj = np.nonzero(ids[:tmax] == e)
        y = R.dense_gemm(x[tt], R.dequant_layer(layer, int(e)))
        for t in ts:                     # rows are disjoint across experts: no write conflicts
            sel = tt < t
            refs[t][tt[sel] * topk + jj[sel]] = y[sel]

    with ThreadPoolExecutor(POOL) as ex:
        list(ex.map(one, used))
    return refs


class _MoE:
    def __init__(self, layer, acts, ts, routes=(True,)):
        self.layer = layer
        p, buf = layers.prepare_layer(layer)
        self.got = {(t, r): _moe_gpu(p, layer, acts, t, with_ws=r) for t in ts for r in routes}
        del buf
        torch.cuda.empty_cache()
        self.ref = _moe_reference(layer, acts, ts)

    def check(self, t, route=True):
        g, r = self.got[(t, route)], self.ref[t]
        assert not np.isnan(r).any(), "every (token, slot) row is routed to a valid expert here"
        err = R.relative_error(g, r)
        assert err <= _tol(self.layer), f"T={t}: relative error {err:.3g} over the whole {g.shape} output"


C4_T = [16, 256, 4096]
C5_T = [64, 1024, 8192]


@pytest.fixture(scope="module")
def c4():
    d = _MoE(*synth.moe_w4a16_mxfp4(t=max(C4_T), experts=128, topk=8, n=4096, k=7168, seed=0), C4_T)
    yield d
    del d


@pytest.mark.timeout(600)
@pytest.mark.parametrize("t", C4_T)
def test_moe_w4a16_mxfp4_e128(c4, t):
    c4.check(t)


@pytest.fixture(scope="module")
def c5():
    d = _MoE(*synth.moe_w4a8_int4(t=max(C5_T), experts=64, topk=6, n=2816, k=4096, seed=0), C5_T)
    yield d
    del d


@pytest.mark.timeout(600)
@pytest.mark.parametrize("t", C5_T)
def test_moe_w4a8_int4_e64_skewed(c5, t):
    c5.check(t)


# ---- whole MoE layers at full size ----------------------------------------------------------
# The layer launches exactly as the benchmark's --layer leg does: tokens are the first T of
# a draw of the largest T, the gate/up align output feeds both products, the down product
# runs with one input row per slot.  Sample: a few tokens (first and last included) x the
# sampled output columns; the oracle computes their gate/up rows in full (SwiGLU needs every
# column), then the sampled columns of the down product and the weighted sum over slots.

def _layer_gpu(up, down, acts, t, act_type):
    topk = acts.topk_ids.shape[1]
    rows, inter = t * topk, down.k
    pu, bu = layers.prepare_layer(up)
    pd, bd = layers.prepare_layer(down)
    bm = qg.moe_block_m(pu, t, topk)
    assert qg.moe_block_m(pd, rows, 1) == bm
    cs, cb = qg.moe_capacity(t, topk, up.experts, bm)
    ids = torch.from_numpy(np.ascontiguousarray(acts.topk_ids[:t], dtype=np.int32)).cuda()
    sid = torch.empty(cs, dtype=torch.int32, device="cuda")
    eid = torch.empty(cb, dtype=torch.int32, device="cuda")
    npp = torch.empty(1, dtype=torch.int32, device="cuda")
    qg.moe_align(ids, t, topk, up.experts, bm, sid, eid, npp)
    x, xs = layers.acts_to_dev(acts)
    x, xs = x[:t], (None if xs is None else xs[:t])
    y1 = torch.empty((rows, 2 * inter), dtype=torch.bfloat16, device="cuda")
    ws1 = torch.zeros(max(1, qg.workspace_bytes(pu, t, topk)), dtype=torch.uint8, device="cuda")
    qg.moe_gemm(pu, x, xs, sid, eid, npp, t, topk, bm, y1, ws1)
    e4, f4 = act_type == "e4m3", act_type == "e2m1"
    if f4:   # SwiGLU -> bf16 -> MXFP4 codes [rows][inter/2] and exponents [rows][inter/32]
        act = torch.empty((rows, inter // 2), dtype=torch.uint8, device="cuda")
        asc = torch.empty((rows, inter // 32), dtype=torch.uint8, device="cuda")
    else:
        act = torch.empty((rows, inter), dtype=torch.uint8 if e4 else torch.bfloat16, device="cuda")
        asc = torch.empty(rows, dtype=torch.float32, device="cuda") if e4 else None
    qg.moe_swiglu(y1, rows, inter, qg.O_BF16, qg.A_FP8_E4M3 if e4 else qg.A_FP4_E2M1 if f4 else qg.A_BF16, act, asc)
    y2 = torch.empty((rows, down.n), dtype=torch.bfloat16, device="cuda")
    ws2 = torch.zeros(max(1, qg.workspace_bytes(pd, rows, 1)), dtype=torch.uint8, device="cuda")
    qg.moe_gemm(pd, act, asc, sid, eid, npp, rows, 1, bm, y2, ws2)
    out = torch.full((t, down.n), float("nan"), dtype=torch.bfloat16, device="cuda")
    w = torch.from_numpy(np.ascontiguousarray(acts.topk_weights[:t])).cuda()
    qg.moe_combine(y2, w, ids, t, topk, up.experts, down.n, qg.O_BF16, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite output"
    return out


@pytest.fixture(scope="module")
def c4_layer():
    up, acts = synth.moe_w4a16_mxfp4(t=4096, experts=128, topk=8, n=4096, k=7168, seed=0)
    down = synth.moe_down_mxfp4(experts=128, n=7168, k=2048, seed=100)
    return up, down, acts


@pytest.mark.parametrize("t", [16, 4096])
def test_moe_layer_mxfp4_e128_full_size(c4_layer, t):
    from oracle import moe_layer as ML
    up, down, acts = c4_layer
    out = _layer_gpu(up, down, acts, t, "bf16")
    rng = np.random.default_rng(t + 5)
    toks = np.unique(np.array([0, t - 1, int(rng.integers(0, t))]))
    cols = _sample(rng, down.n, N_COLS)
    got = layers.out_bits_to_f64(out[torch.from_numpy(toks).cuda()][:, torch.from_numpy(cols).cuda()])
    x = R.activations(synth.Acts(acts.x[toks], None, None), "bf16")
    ref = np.zeros((toks.size, cols.size))
    for i, tk in enumerate(toks):
        for j in range(acts.topk_ids.shape[1]):
            e = int(acts.topk_ids[tk, j])
            h = R.dense_gemm(x[i:i + 1], R.dequant_layer(up, e))
            a = ML.swiglu(h)
            ref[i] += float(acts.topk_weights[tk, j]) * R.dense_gemm(a, R.dequant_rows(down, e, cols))[0]
    err = R.relative_error(got, ref)
    assert err <= TOL16, f"T={t}: relative error {err:.3g}"


@pytest.fixture(scope="module")
def c4_layer_w4a4():
    up, acts = synth.moe_w4a4_mxfp4(t=4096, experts=128, topk=8, n=4096, k=7168, seed=0)
    down = synth.moe_down_w4a4_mxfp4(experts=128, n=7168, k=2048, seed=100)
    return up, down, acts


@pytest.mark.parametrize("t", [16, 4096])
def test_moe_layer_w4a4_e128_full_size(c4_layer_w4a4, t):
    # W4A4 at the MXFP4 layer's shapes: each sampled token's gate/up rows in full (rounded to
    # bfloat16, the product's output type), SwiGLU -> bfloat16 -> MXFP4 in the oracle, then the
    # sampled columns of the down product; the FP8 layers' bar (requantization can move a code)
    from oracle import moe_layer as ML
    from oracle import quant as Q
    up, down, acts = c4_layer_w4a4
    out = _layer_gpu(up, down, acts, t, "e2m1")
    rng = np.random.default_rng(t + 7)
    toks = np.unique(np.array([0, t - 1, int(rng.integers(0, t))]))
    cols = _sample(rng, down.n, N_COLS)
    got = layers.out_bits_to_f64(out[torch.from_numpy(toks).cuda()][:, torch.from_numpy(cols).cuda()])
    x = R.activations(synth.Acts(acts.x[toks], acts.x_scale[toks], None), "e2m1")
    ref = np.zeros((toks.size, cols.size))
    for i, tk in enumerate(toks):
        for j in range(acts.topk_ids.shape[1]):
            e = int(acts.topk_ids[tk, j])
            h = Q.round_to_bf16(R.dense_gemm(x[i:i + 1], R.dequant_layer(up, e)))
            codes, e8 = ML.swiglu_mxfp4(h)
            a = R.activations(synth.Acts(codes, e8, None), "e2m1")
            ref[i] += float(acts.topk_weights[tk, j]) * R.dense_gemm(a, R.dequant_rows(down, e, cols))[0]
    err = R.relative_error(got, ref)
    assert err <= TOL8, f"T={t}: relative error {err:.3g}"


@pytest.mark.parametrize("t", [64, 8192])
def test_moe_w4a8_layer_steps_full_size(t):
    # The W4A8 layer's steps at the benchmark's launch shapes, each on generated inputs:
    # SwiGLU -> e4m3 over T*6 rows of 2*1408, the down product (E=64, N=4096, K=1408, slot
    # rows) and the combine over N=4096.
    from oracle import moe_layer as ML
    from oracle import formats as F
    topk, inter, hidden = 6, 1408, 4096
    _, acts = synth.moe_w4a8_int4(t=t, experts=64, topk=topk, n=64, k=256, seed=0)
    rows = t * topk
    rng = np.random.default_rng(t)
    # SwiGLU -> e4m3
    gu = synth.gate_up_values(rows, inter, "bf16", seed=t)
    codes = torch.empty((rows, inter), dtype=torch.uint8, device="cuda")
    sc = torch.empty(rows, dtype=torch.float32, device="cuda")
    qg.moe_swiglu(torch.from_numpy(gu.view(np.int16)).cuda(), rows, inter, qg.O_BF16, qg.A_FP8_E4M3, codes, sc)
    torch.cuda.synchronize()
    rr = _sample(rng, rows, N_ROWS)
    act, rc, rs = ML.swiglu_e4m3(F.decode_act(gu[rr], "bf16"))
    c_gpu, s_gpu = codes.cpu().numpy()[rr], sc.cpu().numpy()[rr]
    np.testing.assert_allclose(s_gpu, rs, rtol=2.0 ** -20)
    assert np.mean(c_gpu == rc) >= 0.99
    assert R.relative_error(F.decode_e4m3(c_gpu) * s_gpu[:, None].astype(np.float64), act) <= 2.0 ** -4
    # down product on generated e4m3 rows
    down = synth.moe_down_w4a8(experts=64, n=hidden, k=inter, seed=100)
    pd, bd = layers.prepare_layer(down)
    bm = qg.moe_block_m(pd, rows, 1)
    cs, cb = qg.moe_capacity(t, topk, 64, bm)
    ids = torch.from_numpy(np.ascontiguousarray(acts.topk_ids, dtype=np.int32)).cuda()
    sid = torch.empty(cs, dtype=torch.int32, device="cuda")
    eid = torch.empty(cb, dtype=torch.int32, device="cuda")
    npp = torch.empty(1, dtype=torch.int32, device="cuda")
    qg.moe_align(ids, t, topk, 64, bm, sid, eid, npp)
    xq, xs = synth.act_rows(rows, inter, "e4m3", seed=t + 1)
    y2 = torch.full((rows, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(1, qg.workspace_bytes(pd, rows, 1)), dtype=torch.uint8, device="cuda")
    qg.moe_gemm(pd, torch.from_numpy(xq).cuda(), torch.from_numpy(xs).cuda(), sid, eid, npp, rows, 1, bm, y2, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y2).all())
    slots, cols = _sample(rng, rows, N_ROWS), _sample(rng, hidden, N_COLS)
    got = layers.out_bits_to_f64(y2[torch.from_numpy(slots).cuda()][:, torch.from_numpy(cols).cuda()])
    ref = np.empty_like(got)
    for i, sl in enumerate(slots):
        e = int(acts.topk_ids[sl // topk, sl % topk])
        a = F.decode_e4m3(xq[sl:sl + 1]) * float(xs[sl])
        ref[i] = R.dense_gemm(a, R.dequant_rows(down, e, cols))[0]
    assert R.relative_error(got, ref) <= TOL8
    # combine over N = 4096 on generated slot rows and router probabilities
    yv, w, cids = synth.slot_outputs(t, topk, hidden, experts=64, seed=t + 2)
    out = torch.empty((t, hidden), dtype=torch.bfloat16, device="cuda")
    qg.moe_combine(torch.from_numpy(yv.view(np.int16)).cuda(), torch.from_numpy(w).cuda(),
                   torch.from_numpy(cids).cuda(), t, topk, 64, hidden, qg.O_BF16, out)
    torch.cuda.synchronize()
    toks = _sample(rng, t, 8)
    yh = F.decode_act(yv.reshape(t, topk, hidden)[toks], "bf16")
    refc = ML.combine(yh, w[toks], cids[toks], 64)
    gotc = layers.out_bits_to_f64(out[torch.from_numpy(toks).cuda()])
    assert R.relative_error(gotc, refc) <= 2.0 ** -8 + 2.0 ** -16
