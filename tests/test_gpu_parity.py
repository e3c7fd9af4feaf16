"""Parity of the HIP path (through the C ABI) with the CPU oracle, stage by stage and end
to end, at sizes the oracle finishes in seconds (several tiles and ragged tails)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import (assert_attention_close, assert_bf16_within_one_ulp, dev, f64,
                         topk_set_ok)

pytestmark = pytest.mark.gpu

rng = np.random.default_rng(2026)


@pytest.fixture(scope="module")
def H(gpu):
    from long_context_attention_26_amd import hcsa
    return hcsa


def _sync():
    torch.cuda.synchronize()


# ----------------------------------------------------------------------- compression

@pytest.mark.parametrize("ratio,T,D,B", [(4, 4099, 64, 2), (128, 1000, 128, 1), (1, 37, 32, 1),
                                         (3, 200, 256, 3), (128, 128, 128, 2)])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_compress_parity(H, gpu, ratio, T, D, B, io):
    print(f"compress ratio={ratio} T={T} D={D} B={B} io={io}", flush=True)
    tdt = W.torch_dtype(io)
    x = torch.randn(B, T + 5, D, device=gpu).to(tdt)[:, :T]     # sequence stride > T*D
    x = x.contiguous() if B == 1 else x
    xs = torch.empty(B, T + 5, D, device=gpu, dtype=tdt)
    xs[:, :T] = x
    xs = xs[:, :T]
    omega = torch.randn(ratio, device=gpu) / math.sqrt(ratio)
    n = T // ratio
    y = torch.full((B, n + 2, D), float("nan"), device=gpu, dtype=tdt)
    H.compress_kv(xs, omega, ratio, y)
    _sync()
    om = f64(omega)
    alpha = O.pool_weights(om)
    for b in range(B):
        xb = f64(xs[b])
        exact = O.compress(xb, om, ratio)
        got = f64(y[b, :n])
        assert np.isnan(f64(y[b, n:])).all()                    # rows past T//ratio untouched
        # fp32 accumulation error bound of the GPU before its final rounding
        mag = np.abs(xb[: n * ratio].reshape(n, ratio, D)) * alpha[None, :, None]
        acc_err = (ratio + 8) * 2.0 ** -24 * mag.sum(axis=1) + 1e-30
        if io == "f32":
            assert (np.abs(got - exact) <= acc_err).all(), np.abs(got - exact).max()
        else:
            assert_bf16_within_one_ulp(got, O.round_bf16(exact), "compress bf16", acc_err)


def _boundary_distance(v32, e):
    """Distance of |v|/2^e to the nearest e2m1 decision boundary (relative)."""
    t = np.abs(v32) / np.ldexp(1.0, e)
    b = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    return np.min(np.abs(t[..., None] - b), axis=-1) / np.maximum(t, 1e-30)


def test_compress_mxfp4_epilogue(H, gpu):
    B, T, D, r = 2, 4 * 700 + 3, 64, 4
    x = torch.randn(B, T, D, device=gpu).to(torch.bfloat16)
    omega = torch.randn(r, device=gpu) / 2
    n = T // r
    y = torch.zeros(B, n, D // 2, dtype=torch.uint8, device=gpu)
    ys = torch.zeros(B, n, D // 32, dtype=torch.uint8, device=gpu)
    H.compress_kv(x, omega, r, y, ys)
    _sync()
    mism = 0
    for b in range(B):
        # the quantization decision is taken on fp32 values on both sides
        v32 = O.round_fp32(O.compress(f64(x[b]), f64(omega), r))
        codes, se = O.mxfp4_quantize(v32)
        g_codes = O.mxfp4_unpack(y[b].cpu().numpy())
        g_se = ys[b].cpu().numpy().astype(np.int64) - 127
        bad_s = g_se != se
        # a scale can only differ where the block amax sits at a power of two
        amax = np.abs(v32.reshape(n, D // 32, 32)).max(-1)
        ratio_ = amax[bad_s] / np.ldexp(1.0, np.frexp(amax[bad_s])[1] - 1)
        assert (np.minimum(np.abs(ratio_ - 1), np.abs(ratio_ - 2)) < 1e-5).all()
        ok_blocks = np.repeat(~bad_s, 32, axis=1)
        bad_c = (g_codes != codes) & ok_blocks
        near = _boundary_distance(v32, np.repeat(se, 32, axis=1)) < 1e-5
        assert not (bad_c & ~near).any(), "code differs away from a rounding boundary"
        mism += int(bad_c.sum() + bad_s.sum())
    assert mism <= 0.001 * B * n * D


def test_mxfp4_quantize_bit_exact(H, gpu):
    rows, D = 300, 128
    v = rng.standard_normal((rows, D)) * np.exp(rng.uniform(-20, 20, (rows, 1)))
    v[0] = 0.0                                               # all-zero block
    v[1, :32] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4   # exact ties
    v[2, :32] = -np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4) * 2.0 ** -10
    v[3, :32] = 2.0 ** -130                                  # subnormal fp32 amax
    for dt in ("f32", "bf16"):
        vr = O.round_to(v, dt)
        x = dev(vr, W.torch_dtype(dt), gpu)
        packed = torch.zeros(rows, D // 2, dtype=torch.uint8, device=gpu)
        scales = torch.zeros(rows, D // 32, dtype=torch.uint8, device=gpu)
        H.mxfp4_quantize(x, packed, scales)
        _sync()
        codes, se = O.mxfp4_quantize(vr)
        assert np.array_equal(packed.cpu().numpy(), O.mxfp4_pack(codes)), dt
        assert np.array_equal(scales.cpu().numpy().astype(np.int64) - 127, se), dt


# ----------------------------------------------------------------------- top-k

def _scores(shape, kind):
    if kind == "ties":
        return rng.integers(-4, 5, size=shape).astype(np.float64)
    if kind == "zeros":
        s = np.zeros(shape)
        s[..., 1::7] = -0.0
        return s
    return rng.standard_normal(shape) * 3


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("N,k,kind", [(1, 1, "normal"), (5, 64, "normal"), (2047, 64, "ties"),
                                      (2048, 512, "normal"), (2049, 2048, "ties"),
                                      (10000, 1024, "normal"), (7000, 100, "zeros"),
                                      (40000, 4096, "ties")])
def test_topk_bit_exact(H, gpu, sdt, N, k, kind):
    print(f"topk {sdt} N={N} k={k} {kind}", flush=True)
    B, Nq, ratio = 2, 3, 4
    pos0 = max(0, 4 * N - 6)          # rows see N-2 .. N-1 entries (ragged per row)
    s = O.round_to(_scores((B * Nq, N), kind), sdt)
    s[..., ::97] = -np.inf if kind == "normal" else s[..., ::97]
    st = dev(s, W.torch_dtype(sdt), gpu)
    idx = torch.full((B * Nq, k), -7, dtype=torch.int32, device=gpu)
    H.topk(st, B, Nq, N, ratio, pos0, k, idx)
    _sync()
    got = idx.cpu().numpy()
    for r in range(B * Nq):
        nv = O.visible_entries(pos0 + r % Nq, N, ratio)
        want = O.select_topk(s[r], nv, k)
        assert np.array_equal(got[r], want), (r, nv)


@pytest.mark.parametrize("sdt,N,B,Nq,k,kind,pad", [
    ("bf16", 60000, 2, 48, 512, "normal", 0),     # 96 rows, ragged visible counts
    ("bf16", 131072, 1, 64, 1024, "ties", 0),     # the longest rows of this path
    ("f32", 131072, 1, 64, 300, "normal", 0),
    ("bf16", 66560, 1, 64, 512, "normal", 0),     # a prefill chunk's row length
    ("f32", 32767, 1, 70, 300, "normal", 3),      # ragged last chunk, unaligned stride
    ("bf16", 9001, 1, 64, 700, "ties", 1),
    ("bf16", 9001, 1, 64, 100, "normal", 1),
    ("bf16", 20000, 1, 64, 777, "zeros", 0),      # every key tied
    ("f32", 5000, 3, 40, 4096, "ties", 0),        # k near the visible count
    ("bf16", 3000, 1, 64, 4096, "normal", 0),     # k above it: every visible entry, then -1
    ("bf16", 2000, 1, 100, 1, "normal", 0),
])
def test_topk_many_rows_bit_exact(H, gpu, sdt, N, B, Nq, k, kind, pad):
    """Many short rows (prefill): one block per row holds the row's keys on chip."""
    print(f"topk rows {sdt} N={N} B={B} Nq={Nq} k={k} {kind}", flush=True)
    ratio = 4
    pos0 = 4 * N - 2 * Nq                 # visible counts from N - Nq/2 up to N, capped
    s = O.round_to(_scores((B * Nq, N), kind), sdt)
    if kind == "normal":
        s[..., ::89] = -np.inf
    st = dev(s, W.torch_dtype(sdt), gpu)
    assert H.topk_workspace_size(H.dtype_code(st), B, Nq, N, k) == 0
    over = 131073                                     # one past this path's row limit
    assert H.topk_workspace_size(H.dtype_code(st), B, Nq, over, k) > 0
    if pad:                               # unaligned row stride: element loads
        wide = torch.zeros(B * Nq, N + pad, dtype=st.dtype, device=gpu)
        wide[:, :N] = st
        st = wide[:, :N]
    idx = torch.full((B * Nq, k), -7, dtype=torch.int32, device=gpu)
    H.topk(st, B, Nq, N, ratio, pos0, k, idx)
    _sync()
    got = idx.cpu().numpy()
    for r in range(B * Nq):
        nv = O.visible_entries(pos0 + r % Nq, N, ratio)
        want = O.select_topk(s[r], nv, k)
        assert np.array_equal(got[r], want), (r, nv)


@pytest.mark.parametrize("sdt,N,rows,k,kind", [
    ("bf16", 262144, 4, 1024, "normal"),       # decode rows: segment lists
    ("bf16", 262144, 2, 1024, "skewed"),       # the top keys crowd one segment: exact fallback
    ("f32", 100000, 3, 500, "normal"),
    ("bf16", 8193, 2, 10, "normal"),           # second segment holds one key
    ("f32", 30000, 5, 4096, "ties"),
])
def test_topk_long_rows_bit_exact(H, gpu, sdt, N, rows, k, kind):
    """Few long rows (decode): per-segment candidate lists, then one resolve block per row."""
    print(f"topk segments {sdt} N={N} rows={rows} k={k} {kind}", flush=True)
    ratio, pos0 = 4, 4 * N - 1                  # every row sees all N entries
    base = rng.standard_normal((rows, N)) * 3 if kind != "ties" else _scores((rows, N), "ties")
    if kind == "skewed":
        base[:, 100000:108000] += 40.0
    s = O.round_to(base, sdt)
    st = dev(s, W.torch_dtype(sdt), gpu)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=gpu)
    H.topk(st, rows, 1, N, ratio, pos0, k, idx)
    _sync()
    got = idx.cpu().numpy()
    for r in range(rows):
        assert np.array_equal(got[r], O.select_topk(s[r], N, k)), r


def test_topk_deterministic(H, gpu):
    s = dev(O.round_bf16(rng.integers(0, 3, size=(1, 262144)).astype(float)), torch.bfloat16, gpu)
    outs = []
    for _ in range(3):
        idx = torch.empty(1, 1024, dtype=torch.int32, device=gpu)
        H.topk(s, 1, 1, 262144, 1, 262143, 1024, idx)
        outs.append(idx.cpu().numpy())
    assert all(np.array_equal(outs[0], o) for o in outs)
    assert np.array_equal(outs[0][0], O.select_topk(f64(s)[0], 262144, 1024))


# ----------------------------------------------------------------------- indexer

@pytest.mark.parametrize("case", [
    dict(kdt="f32", H_I=1, d_I=32, N=1024, Nq=1, B=1, k=64, sdt="f32"),
    dict(kdt="bf16", H_I=4, d_I=64, N=5000, Nq=1, B=3, k=512, sdt="bf16"),
    dict(kdt="bf16", H_I=4, d_I=64, N=3000, Nq=5, B=1, k=128, sdt="f32"),
    dict(kdt="bf16", H_I=2, d_I=128, N=2100, Nq=2, B=2, k=64, sdt="bf16"),
    dict(kdt="mxfp4", H_I=4, d_I=64, N=4500, Nq=1, B=2, k=256, sdt="bf16"),
    dict(kdt="mxfp4", H_I=1, d_I=32, N=900, Nq=3, B=1, k=64, sdt="f32"),
    dict(kdt="mxfp4", H_I=8, d_I=128, N=3000, Nq=2, B=2, k=100, sdt="f32"),
    dict(kdt="mxfp4", H_I=16, d_I=64, N=1500, Nq=1, B=1, k=200, sdt="bf16"),
    # many query tokens per sequence: the prefill GEMM kernel
    dict(kdt="bf16", H_I=4, d_I=64, N=3000, Nq=64, B=2, k=256, sdt="bf16"),
    dict(kdt="bf16", H_I=2, d_I=128, N=2000, Nq=64, B=1, k=100, sdt="f32"),
    dict(kdt="bf16", H_I=1, d_I=64, N=5000, Nq=384, B=1, k=512, sdt="bf16"),
    dict(kdt="bf16", H_I=4, d_I=32, N=4100, Nq=256, B=2, k=300, sdt="bf16"),
    dict(kdt="bf16", H_I=4, d_I=64, N=8000, Nq=512, B=2, k=512, sdt="bf16"),
    dict(kdt="bf16", H_I=2, d_I=64, N=2500, Nq=96, B=1, k=64, sdt="f32"),   # wave kernel
])
def test_index_scores_and_topk(H, gpu, case):
    print(f"indexer {case}", flush=True)
    B, Nq, H_I, d_I, N, k = case["B"], case["Nq"], case["H_I"], case["d_I"], case["N"], case["k"]
    ratio = 4
    pos0 = 4 * N - Nq                            # the last rows see all N entries
    qdt = "f32" if case["kdt"] == "f32" else "bf16"
    q = O.round_to(rng.standard_normal((B, Nq, H_I, d_I)), qdt)
    w = O.round_fp32(rng.standard_normal((B, Nq, H_I)))      # signed weights
    keys = O.round_to(rng.standard_normal((B, N + 3, d_I)), qdt)
    qt = dev(q, W.torch_dtype(qdt), gpu)
    wt = dev(w, torch.float32, gpu)
    if case["kdt"] == "mxfp4":
        codes, se = O.mxfp4_quantize(keys)
        kt = torch.from_numpy(O.mxfp4_pack(codes)).to(gpu)
        kst = torch.from_numpy((se + 127).astype(np.uint8)).to(gpu)
        keys_seen = O.mxfp4_dequantize(codes, se)
        q_seen = O.mxfp4_roundtrip(q)
    else:
        kt = dev(keys, W.torch_dtype(qdt), gpu)
        kst = None
        keys_seen, q_seen = keys, q
    sdt = H.BF16 if case["sdt"] == "bf16" else H.F32
    scores = torch.zeros(B * Nq, N, device=gpu, dtype=W.torch_dtype(case["sdt"]))
    idx = torch.empty(B, Nq, k, dtype=torch.int32, device=gpu)
    H.csa_index_topk(qt, wt, kt, N, ratio, pos0, k, sdt, idx, k_scales=kst, scores_out=scores)
    # scoring and selection as two calls give the same result
    ws = H.alloc_workspace(H.topk_workspace_size(sdt, B, Nq, N, k), gpu)
    scores2 = torch.zeros_like(scores)
    idx2 = torch.empty_like(idx)
    H.csa_index_scores(qt, wt, kt, N, ratio, pos0, scores2, k_scales=kst)
    H.topk(scores2, B, Nq, N, ratio, pos0, k, idx2.view(B * Nq, k), ws)
    _sync()
    assert torch.equal(scores, scores2) and torch.equal(idx, idx2)
    gs = f64(scores)
    gi = idx.cpu().numpy().reshape(B * Nq, k)
    for b in range(B):
        for i in range(Nq):
            r = b * Nq + i
            nv = O.visible_entries(pos0 + i, N, ratio)
            exact = O.index_scores(q_seen[b, i], w[b, i], keys_seen[b], nv, "f32")
            # fp32 error bound of the GPU's sums: (d_I + H_I + 4) roundings of sum |terms|
            mag = (np.abs(keys_seen[b, :nv]) @ np.abs(q_seen[b, i]).T) @ np.abs(w[b, i])
            acc_err = (d_I + H_I + 4) * 2.0 ** -24 * mag + 1e-30
            if case["sdt"] == "f32":
                err = np.abs(gs[r, :nv] - exact)
                assert (err <= acc_err).all(), (err / acc_err).max()
            else:
                ref16 = O.round_bf16(exact)
                assert_bf16_within_one_ulp(gs[r, :nv], ref16, "bf16 scores", acc_err)
            # selection on the GPU's own score array is bit-exact
            assert np.array_equal(gi[r], O.select_topk(gs[r], nv, k)), r
            # and against the exact scores it differs only at the threshold
            ref_scores = exact if case["sdt"] == "f32" else O.round_bf16(exact)
            topk_set_ok(gi[r], O.select_topk(ref_scores, nv, k), exact, k, "indexer e2e",
                        rel=2e-2 if case["sdt"] == "bf16" else 1e-5)


@pytest.mark.parametrize("case", [
    # 16 sequences x 262144 entries
    dict(B=16, Nq=1, N=262144, H_I=4, d_I=64, k=1024, sdt="bf16", kind="normal"),
    # ragged visible counts (several query tokens per sequence), fp32 scores, 2 MFMA steps
    dict(B=3, Nq=5, N=150001, H_I=8, d_I=128, k=700, sdt="f32", kind="normal"),
    # a run of identical keys far above the rest: lists overflow, exact full-row fallback
    dict(B=8, Nq=1, N=200000, H_I=4, d_I=64, k=1024, sdt="bf16", kind="crowd"),
    # every key identical: all scores tie, the lowest indices win
    dict(B=4, Nq=1, N=70000, H_I=2, d_I=32, k=512, sdt="bf16", kind="equal"),
])
def test_mx_index_topk_long_rows(H, gpu, case):
    """MXFP4 keys, long rows at the decode workload's scale (segment candidate lists, the
    exact fallback on overflow, all-equal rows): the one-call form equals the two-call form
    bit for bit, and the selection on the GPU's own score array equals the oracle's."""
    print(f"mx index+topk {case}", flush=True)
    B, Nq, N, H_I, d_I, k = case["B"], case["Nq"], case["N"], case["H_I"], case["d_I"], case["k"]
    ratio, pos0 = 4, 4 * N - Nq
    g = torch.Generator().manual_seed(7)
    codes = torch.randint(0, 256, (B, N, d_I // 2), generator=g, dtype=torch.uint8)
    scl = torch.randint(121, 128, (B, N, d_I // 32), generator=g, dtype=torch.uint8)
    if case["kind"] == "crowd":
        codes[:, 50000:60000] = 0x77                  # every element +6: the largest scores
        scl[:, 50000:60000] = 127
    if case["kind"] == "equal":
        codes[:] = 0x22
        scl[:] = 127
    q = torch.randn(B, Nq, H_I, d_I, generator=g).to(torch.bfloat16)
    if case["kind"] in ("crowd", "equal"):
        q = q.abs()                                   # positive dots with the all-positive keys
    w = torch.rand(B, Nq, H_I, generator=g) + 0.1
    kt, kst, qt, wt = codes.to(gpu), scl.to(gpu), q.to(gpu), w.to(gpu)
    sdt = H.BF16 if case["sdt"] == "bf16" else H.F32
    sdtype = W.torch_dtype(case["sdt"])
    scores = torch.zeros(B * Nq, N, device=gpu, dtype=sdtype)
    idx = torch.full((B, Nq, k), -7, dtype=torch.int32, device=gpu)
    H.csa_index_topk(qt, wt, kt, N, ratio, pos0, k, sdt, idx, k_scales=kst, scores_out=scores)
    ws = H.alloc_workspace(H.topk_workspace_size(sdt, B, Nq, N, k), gpu)
    scores2 = torch.zeros_like(scores)
    idx2 = torch.empty_like(idx)
    H.csa_index_scores(qt, wt, kt, N, ratio, pos0, scores2, k_scales=kst)
    H.topk(scores2, B, Nq, N, ratio, pos0, k, idx2.view(B * Nq, k), ws)
    _sync()
    assert torch.equal(scores, scores2)
    assert torch.equal(idx, idx2)
    gs = f64(scores)
    gi = idx.cpu().numpy().reshape(B * Nq, k)
    for r in sorted({0, B * Nq - 1, (B * Nq) // 2}):
        nv = O.visible_entries(pos0 + r % Nq, N, ratio)
        assert np.array_equal(gi[r], O.select_topk(gs[r], nv, k)), r
    if case["kind"] == "equal":
        assert (gs[:, :1] == gs[:, : N - Nq]).all()
        assert np.array_equal(gi[0], np.arange(k))


@pytest.mark.parametrize("case", [
    # the chunked-prefill shape: 4096 query tokens x 4 heads against 66560 entries
    dict(B=1, Nq=4096, N=66560, H_I=4, d_I=64, k=512, sdt="bf16", kind="normal"),
    # two sequences, fp32 scores, d_I 128, ragged causal edges inside the key chunks
    dict(B=2, Nq=256, N=9000, H_I=2, d_I=128, k=300, sdt="f32", kind="normal"),
    # one query head (32 tokens per wave); k at or above the visible count of the first rows
    # (all taken), and for the others every visible key is a candidate (short rows)
    dict(B=1, Nq=128, N=1500, H_I=1, d_I=32, k=1480, sdt="bf16", kind="normal"),
    # a run of identical keys far above the rest: candidate lists overflow, exact path
    dict(B=1, Nq=512, N=40000, H_I=4, d_I=64, k=512, sdt="bf16", kind="crowd"),
])
def test_gemm_index_topk_prefill_scale(H, gpu, case):
    """Prefill shapes at the chunked-prefill scale (the GEMM scan, the one-block-per-row
    selector with its list overflow and take-all cases): the one-call form equals scoring and
    selecting in two calls bit for bit, and the selection on the GPU's own score array equals
    the oracle's."""
    print(f"gemm index+topk {case}", flush=True)
    B, Nq, N, H_I, d_I, k = case["B"], case["Nq"], case["N"], case["H_I"], case["d_I"], case["k"]
    ratio = 4
    pos0 = 4 * N - Nq - 37 if case["kind"] != "crowd" else 4 * N - Nq   # ragged: early rows see fewer
    g = torch.Generator().manual_seed(11)
    keys = torch.randn(B, N, d_I, generator=g)
    if case["kind"] == "crowd":
        keys[:, 20000:24000] = 3.0
    q = torch.randn(B, Nq, H_I, d_I, generator=g)
    if case["kind"] == "crowd":
        q = q.abs()
    w = torch.rand(B, Nq, H_I, generator=g) + 0.1
    kt = keys.to(torch.bfloat16).to(gpu)
    qt = q.to(torch.bfloat16).to(gpu)
    wt = w.to(gpu)
    sdt = H.BF16 if case["sdt"] == "bf16" else H.F32
    sdtype = W.torch_dtype(case["sdt"])
    scores = torch.zeros(B * Nq, N, device=gpu, dtype=sdtype)
    idx = torch.full((B, Nq, k), -7, dtype=torch.int32, device=gpu)
    H.csa_index_topk(qt, wt, kt, N, ratio, pos0, k, sdt, idx, scores_out=scores)
    ws = H.alloc_workspace(H.topk_workspace_size(sdt, B, Nq, N, k), gpu)
    scores2 = torch.zeros_like(scores)
    idx2 = torch.empty_like(idx)
    H.csa_index_scores(qt, wt, kt, N, ratio, pos0, scores2)
    H.topk(scores2, B, Nq, N, ratio, pos0, k, idx2.view(B * Nq, k), ws)
    _sync()
    assert torch.equal(scores, scores2)
    assert torch.equal(idx, idx2)
    gi = idx.cpu().numpy().reshape(B * Nq, k)
    rows = sorted({0, 1, 63, Nq - 1, B * Nq - 1, (B * Nq) // 2})
    gs = f64(scores[rows])
    for r, srow in zip(rows, gs):
        nv = O.visible_entries(pos0 + r % Nq, N, ratio)
        assert np.array_equal(gi[r], O.select_topk(srow, nv, k)), r


# ----------------------------------------------------------------------- attention

def _attn_inputs(B, Nq, Hh, d, N, T_raw, dt):
    q = O.round_to(rng.standard_normal((B, Nq, Hh, d)), dt)
    Kc = O.round_to(rng.standard_normal((B, N, d)), dt)
    Vc = O.round_to(rng.standard_normal((B, N, d)), dt)
    Kr = O.round_to(rng.standard_normal((B, T_raw, d)), dt)
    Vr = O.round_to(rng.standard_normal((B, T_raw, d)), dt)
    return q, Kc, Vc, Kr, Vr


@pytest.mark.parametrize("case", [
    dict(dt="f32", H=1, d=64, N=1024, k=64, n_win=128, Nq=1, B=1, pos0=4095),      # config 1 shape
    dict(dt="bf16", H=16, d=128, N=3000, k=512, n_win=128, Nq=1, B=3, pos0=11999),  # MFMA path
    dict(dt="bf16", H=16, d=128, N=600, k=1024, n_win=128, Nq=1, B=1, pos0=2399),   # k > n_c: padding
    dict(dt="bf16", H=16, d=128, N=2000, k=256, n_win=128, Nq=40, B=1, pos0=7900),  # prefill rows
    dict(dt="bf16", H=4, d=64, N=700, k=100, n_win=50, Nq=2, B=2, pos0=2798),       # generic bf16
    dict(dt="bf16", H=16, d=128, N=10, k=16, n_win=128, Nq=1, B=1, pos0=40),        # window clipped at 0
    dict(dt="f32", H=2, d=32, N=100, k=0, n_win=0, Nq=1, B=1, pos0=399),            # empty key list
    dict(dt="bf16", H=16, d=128, N=100, k=0, n_win=0, Nq=1, B=1, pos0=399),         # empty, MFMA
])
def test_csa_sparse_attention(H, gpu, case):
    print(f"csa {case}", flush=True)
    B, Nq, Hh, d, N, k, w = case["B"], case["Nq"], case["H"], case["d"], case["N"], case["k"], case["n_win"]
    pos0, dt, ratio = case["pos0"], case["dt"], 4
    raw_pos0 = max(0, pos0 - w - 5)
    T_raw = pos0 + Nq - raw_pos0 + 3
    q, Kc, Vc, Kr, Vr = _attn_inputs(B, Nq, Hh, d, N, T_raw, dt)
    idx = np.full((B, Nq, k), -1, dtype=np.int64)
    for b in range(B):
        for i in range(Nq):
            nv = O.visible_entries(pos0 + i, N, ratio)
            idx[b, i] = O.select_topk(rng.standard_normal(N), nv, k) if k else idx[b, i]
    tdt = W.torch_dtype(dt)
    out = torch.full((B, Nq, Hh, d), float("nan"), device=gpu)
    lse = torch.full((B, Nq, Hh), float("nan"), device=gpu)
    H.csa_sparse_attn(dev(q, tdt, gpu), dev(Kc, tdt, gpu), dev(Vc, tdt, gpu), N,
                      torch.from_numpy(idx.astype(np.int32)).to(gpu), dev(Kr, tdt, gpu),
                      dev(Vr, tdt, gpu), raw_pos0, w, ratio, pos0, 1 / math.sqrt(d), out, lse)
    _sync()
    go, gl = f64(out), f64(lse)
    ro, rl = np.zeros_like(go), np.zeros_like(gl)
    for b in range(B):
        for i in range(Nq):
            ro[b, i], rl[b, i] = O.csa_attention(q[b, i], Kc[b], Vc[b], idx[b, i], Kr[b], Vr[b],
                                                 raw_pos0, pos0 + i, w, 1 / math.sqrt(d), ratio)
    assert_attention_close(go, gl, ro, rl, dt == "f32", f"csa {case}")


@pytest.mark.parametrize("case", [
    dict(dt="f32", H=1, d=64, N=32, Nq=1, B=1, pos0=4095),           # config 1 shape
    dict(dt="bf16", H=16, d=128, N=1024, Nq=1, B=2, pos0=131071),     # config 2 shape
    dict(dt="bf16", H=16, d=128, N=5000, Nq=1, B=1, pos0=640000 - 1), # many splits
    dict(dt="bf16", H=16, d=128, N=40, Nq=300, B=1, pos0=4900),       # causal prefill rows
    dict(dt="bf16", H=16, d=128, N=2100, Nq=64, B=2, pos0=128 * 2000 - 30),  # 16-token tiles
    dict(dt="bf16", H=16, d=128, N=8, Nq=40, B=1, pos0=100),          # tiles partly empty
    dict(dt="bf16", H=16, d=128, N=300, Nq=33, B=3, pos0=128 * 290),  # ragged last tile
    dict(dt="bf16", H=8, d=64, N=50, Nq=3, B=2, pos0=6399),           # generic path
    dict(dt="bf16", H=16, d=128, N=8, Nq=2, B=1, pos0=100),           # nothing visible
])
def test_hca_dense_attention(H, gpu, case):
    print(f"hca {case}", flush=True)
    B, Nq, Hh, d, N, pos0, dt = case["B"], case["Nq"], case["H"], case["d"], case["N"], case["pos0"], case["dt"]
    ratio = 128
    q, Kh, Vh, _, _ = _attn_inputs(B, Nq, Hh, d, N, 1, dt)
    tdt = W.torch_dtype(dt)
    out = torch.full((B, Nq, Hh, d), float("nan"), device=gpu)
    lse = torch.full((B, Nq, Hh), float("nan"), device=gpu)
    H.hca_dense_attn(dev(q, tdt, gpu), dev(Kh, tdt, gpu), dev(Vh, tdt, gpu), N, ratio, pos0,
                     1 / math.sqrt(d), out, lse)
    _sync()
    go, gl = f64(out), f64(lse)
    ro, rl = np.zeros_like(go), np.zeros_like(gl)
    for b in range(B):
        for i in range(Nq):
            ro[b, i], rl[b, i] = O.hca_attention(q[b, i], Kh[b], Vh[b], pos0 + i, 1 / math.sqrt(d), ratio)
    assert_attention_close(go, gl, ro, rl, dt == "f32", f"hca {case}")


@pytest.mark.parametrize("kind", ["csa", "hca", "csa+hca"])
def test_attention_deterministic_and_split_invariant(H, gpu, kind):
    """Split counts 1, 2, 7 and 64 of each query's key list (hcsa_set_attn_splits; 64
    takes the merge's LDS-weight form, 7 and 2 its register form, 1 no merge): every count
    agrees with the others and with the oracle, and repeating a call gives the same bits."""
    print(f"split invariance {kind}", flush=True)
    B, Nq, Hh, d, N, Nh, k, w, ratio = 2, 1, 16, 128, 3000, 90, 1024, 128, 4
    pos0 = 128 * Nh - 1
    scale = 1 / math.sqrt(d)
    q, Kc, Vc, Kr, Vr = _attn_inputs(B, Nq, Hh, d, N, pos0 + 1, "bf16")
    _, Kh, Vh, _, _ = _attn_inputs(B, Nq, Hh, d, Nh, 1, "bf16")
    idx = np.stack([O.select_topk(rng.standard_normal(N), O.visible_entries(pos0, N, ratio), k)
                    for _ in range(B)])[:, None, :]
    t = lambda a: dev(a, torch.bfloat16, gpu)
    args_c = dict(q=t(q), kc=t(Kc), vc=t(Vc), idx=torch.from_numpy(idx.astype(np.int32)).to(gpu),
                  kr=t(Kr), vr=t(Vr))
    kh, vh = t(Kh), t(Vh)
    ref = {}
    for b in range(B):
        ref[("c", b)] = O.csa_attention(q[b, 0], Kc[b], Vc[b], idx[b, 0], Kr[b], Vr[b], 0, pos0,
                                        w, scale, ratio)
        ref[("h", b)] = O.hca_attention(q[b, 0], Kh[b], Vh[b], pos0, scale, 128)

    def run(splits):
        H.set_attn_splits(splits)
        try:
            oc, lc = torch.empty(B, Nq, Hh, d, device=gpu), torch.empty(B, Nq, Hh, device=gpu)
            oh, lh = torch.empty_like(oc), torch.empty_like(lc)
            if kind == "csa":
                H.csa_sparse_attn(args_c["q"], args_c["kc"], args_c["vc"], N, args_c["idx"],
                                  args_c["kr"], args_c["vr"], 0, w, ratio, pos0, scale, oc, lc)
            elif kind == "hca":
                H.hca_dense_attn(args_c["q"], kh, vh, Nh, 128, pos0, scale, oh, lh)
            else:
                H.csa_hca_attn(args_c["q"], args_c["kc"], args_c["vc"], N, args_c["idx"],
                               args_c["kr"], args_c["vr"], 0, w, ratio, kh, vh, Nh, 128, pos0,
                               scale, oc, lc, oh, lh)
            _sync()
        finally:
            H.set_attn_splits(0)
        return [x.cpu() for x in (oc, lc, oh, lh)]

    results = {}
    for splits in (1, 2, 7, 64):
        a, b2 = run(splits), run(splits)
        for x, y in zip(a, b2):
            assert torch.equal(x, y), f"{kind}: splits {splits} not deterministic"
        results[splits] = a
        for b in range(B):
            if kind != "hca":
                assert_attention_close(f64(a[0][b]), f64(a[1][b]), ref[("c", b)][0][None],
                                       ref[("c", b)][1][None], False, f"csa splits {splits}")
            if kind != "csa":
                assert_attention_close(f64(a[2][b]), f64(a[3][b]), ref[("h", b)][0][None],
                                       ref[("h", b)][1][None], False, f"hca splits {splits}")
    # Between split counts only roundings differ: the P.V product takes the probabilities
    # as bf16, each split rounding them relative to its own running maximum (relative error
    # <= 2^-9 per term on each side), and the fp32 sums run in another order.  So
    # |do| <= 2^-8 sum_j p_j |v_j| / sum_j p_j (+ fp32 slack) per output; lse (fp32 sums of
    # unrounded probabilities) within 1e-5.
    def abs_weighted(b, csa):
        if csa:
            n_vis = O.visible_entries(pos0, N, ratio)
            keys, vals = O.csa_keys(Kc[b], Vc[b], idx[b, 0], Kr[b], Vr[b], 0, pos0, w, n_vis)
        else:
            n = O.visible_entries(pos0, Nh, 128)
            keys, vals = Kh[b][:n], Vh[b][:n]
        return O.softmax_weights(q[b, 0], keys, scale) @ np.abs(vals)     # [H, d]

    base = results[1]
    for splits in (2, 7, 64):
        for which, (x, y) in enumerate(zip(base, results[splits])):
            if (kind == "csa" and which >= 2) or (kind == "hca" and which < 2):
                continue
            xf, yf = f64(x), f64(y)
            if which % 2 == 1:                        # lse
                assert np.abs(xf - yf).max() <= 1e-5, f"{kind}: lse, splits 1 vs {splits}"
                continue
            for b in range(B):
                bound = 2.0 ** -8 * abs_weighted(b, which == 0) + 1e-6
                err = np.abs(xf[b, 0] - yf[b, 0])
                assert (err <= bound).all(), \
                    f"{kind}: splits 1 vs {splits}, output {which}, worst {(err / bound).max()}"
    with pytest.raises(H.HcsaError):
        H.set_attn_splits(-1)


def test_compress_batched_equals_single_calls(H, gpu):
    """The batched pooling launch gives bit-identical results to one call per job."""
    B, T = 3, 1000
    K = torch.randn(B, T, 128, device=gpu).to(torch.bfloat16)
    I = torch.randn(B, T, 64, device=gpu).to(torch.bfloat16)
    F = torch.randn(B, T, 32, device=gpu)
    om4, om128 = torch.randn(4, device=gpu), torch.randn(128, device=gpu)
    outs_a = [torch.zeros(B, T // 4, 128, device=gpu, dtype=torch.bfloat16),
              torch.zeros(B, T // 4, 32, dtype=torch.uint8, device=gpu),
              torch.zeros(B, T // 4, 2, dtype=torch.uint8, device=gpu),
              torch.zeros(B, T // 128, 128, device=gpu, dtype=torch.bfloat16),
              torch.zeros(B, T // 4, 32, device=gpu)]
    outs_b = [torch.ones_like(t) for t in outs_a]
    H.compress_kv(K, om4, 4, outs_a[0])
    H.compress_kv(I, om4, 4, outs_a[1], outs_a[2])
    H.compress_kv(K, om128, 128, outs_a[3])
    H.compress_kv(F, om4, 4, outs_a[4])
    jobs = [H.pool_job(K, om4, 4, outs_b[0]), H.pool_job(I, om4, 4, outs_b[1], outs_b[2]),
            H.pool_job(K, om128, 128, outs_b[3]), H.pool_job(F, om4, 4, outs_b[4])]
    H.compress_kv_batched(jobs, B)
    _sync()
    for a, b in zip(outs_a, outs_b):
        assert torch.equal(a, b)
    with pytest.raises(H.HcsaError):
        H.compress_kv_batched([H.pool_job(K, om4, 3, outs_b[0])] * 9, B)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_topk_massive_ties_take_lowest_indices(H, gpu, sdt):
    """More tied candidates than the selector's candidate list holds: the exact full-row
    resolution still returns the lowest indices."""
    N, k = 50000, 777
    s = np.zeros((2, N))
    s[1, ::3] = 1.0                                     # row 1: 16667 tied maxima
    st = dev(s, W.torch_dtype(sdt), gpu)
    idx = torch.empty(2, k, dtype=torch.int32, device=gpu)
    H.topk(st, 2, 1, N, 1, N - 1, k, idx)
    _sync()
    got = idx.cpu().numpy()
    assert np.array_equal(got[0], np.arange(k))
    assert np.array_equal(got[1], np.arange(0, 3 * k, 3))
    for r in range(2):
        assert np.array_equal(got[r], O.select_topk(s[r], N, k))
