"""Ragged batches: every sequence of a call at its own position (per-sequence positions in
device memory).  Each stage against the oracle per sequence, and the batched call against
one call per sequence at that sequence's position (scores and selection bit for bit)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import assert_attention_close, assert_bf16_within_one_ulp, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H(gpu):
    from long_context_attention_26_amd import hcsa
    return hcsa


CASES = [
    # decode, one token per sequence: wave indexer, segmented top-k, decode HCA, split-K CSA
    dict(name="decode-bf16", Nq=1, pos=[69999, 12345, 40077, 9001], H_I=4, d_I=64, kdt="bf16",
         sdt="bf16", k=512, dt="bf16", H=16, d=128),
    # decode with MXFP4 indexer keys (scaled fp4 MFMA scan)
    dict(name="decode-mxfp4", Nq=1, pos=[30000, 5000, 20003], H_I=4, d_I=64, kdt="mxfp4",
         sdt="bf16", k=256, dt="bf16", H=16, d=128),
    # chunked prefill, 64 tokens per sequence at different offsets: GEMM indexer, one block
    # per row top-k, 16-token HCA tiles, CSA prefill rows
    dict(name="prefill", Nq=64, pos=[20000, 3001, 12800], H_I=4, d_I=64, kdt="bf16",
         sdt="bf16", k=300, dt="bf16", H=16, d=128),
    # fp32 throughout: the generic kernels
    dict(name="f32", Nq=2, pos=[4095, 1000, 2222], H_I=1, d_I=32, kdt="f32", sdt="f32", k=64,
         dt="f32", H=1, d=64),
]


def _keys(case, B, N, gen, gpu):
    """Indexer keys on the GPU and the values the kernels see (host, float64)."""
    d_I = case["d_I"]
    keys = torch.randn(B, N, d_I, generator=gen, dtype=torch.float32)
    if case["kdt"] == "mxfp4":
        codes, se = O.mxfp4_quantize(keys.double().numpy())
        kt = torch.from_numpy(O.mxfp4_pack(codes)).to(gpu)
        kst = torch.from_numpy((se + 127).astype(np.uint8)).to(gpu)
        return kt, kst, O.mxfp4_dequantize(codes, se)
    kt = keys.to(W.torch_dtype(case["kdt"]))
    return kt.to(gpu), None, f64(kt)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_ragged_batch(H, gpu, case):
    print(f"ragged {case['name']}", flush=True)
    pos = case["pos"]
    B, Nq, H_I, d_I, k = len(pos), case["Nq"], case["H_I"], case["d_I"], case["k"]
    Hh, d, n_win, scale = case["H"], case["d"], 128, 1 / math.sqrt(case["d"])
    top = max(pos) + Nq                            # one past the last query position
    N, N_h, T_raw = top // 4, top // 128 + 1, top
    gen = torch.Generator().manual_seed(5)
    seq_pos = torch.tensor(pos, dtype=torch.int64, device=gpu)
    tdt = W.torch_dtype(case["dt"])

    # ---- indexer + top-k: batched ragged call, and one call per sequence
    qdt = "f32" if case["kdt"] == "f32" else "bf16"
    qi = torch.randn(B, Nq, H_I, d_I, generator=gen).to(W.torch_dtype(qdt))
    wi = torch.rand(B, Nq, H_I, generator=gen) + 0.1
    kt, kst, keys_seen = _keys(case, B, N, gen, gpu)
    qit, wit = qi.to(gpu), wi.to(gpu)
    sdt = H.BF16 if case["sdt"] == "bf16" else H.F32
    scores = torch.zeros(B * Nq, N, device=gpu, dtype=W.torch_dtype(case["sdt"]))
    idx = torch.full((B, Nq, k), -7, dtype=torch.int32, device=gpu)
    H.csa_index_topk(qit, wit, kt, N, 4, 0, k, sdt, idx, k_scales=kst, scores_out=scores,
                     seq_pos=seq_pos)
    for b in range(B):
        s1 = torch.zeros(Nq, N, device=gpu, dtype=scores.dtype)
        i1 = torch.full((1, Nq, k), -7, dtype=torch.int32, device=gpu)
        H.csa_index_topk(qit[b:b + 1], wit[b:b + 1], kt[b:b + 1], N, 4, pos[b], k, sdt, i1,
                         k_scales=None if kst is None else kst[b:b + 1], scores_out=s1)
        torch.cuda.synchronize()
        assert torch.equal(i1[0], idx[b]), f"sequence {b}: batched selection differs"
        for i in range(Nq):
            nv = O.visible_entries(pos[b] + i, N, 4)
            assert torch.equal(s1[i, :nv], scores[b * Nq + i, :nv]), f"sequence {b} row {i}"

    # against the oracle: scores within the accumulation bound, selection bit for bit on the
    # GPU's own scores
    gs = f64(scores)
    gi = idx.cpu().numpy().reshape(B * Nq, k)
    q_seen = O.mxfp4_roundtrip(f64(qi)) if case["kdt"] == "mxfp4" else f64(qi)
    w64 = f64(wi)
    for b in range(B):
        for i in sorted({0, Nq - 1}):
            r = b * Nq + i
            nv = O.visible_entries(pos[b] + i, N, 4)
            exact = O.index_scores(q_seen[b, i], w64[b, i], keys_seen[b], nv, "f32")
            mag = (np.abs(keys_seen[b, :nv]) @ np.abs(q_seen[b, i]).T) @ np.abs(w64[b, i])
            acc_err = (d_I + H_I + 4) * 2.0 ** -24 * mag + 1e-30
            if case["sdt"] == "f32":
                assert (np.abs(gs[r, :nv] - exact) <= acc_err).all()
            else:
                assert_bf16_within_one_ulp(gs[r, :nv], O.round_bf16(exact), "bf16 scores", acc_err)
            assert np.array_equal(gi[r], O.select_topk(gs[r], nv, k)), (b, i)

    # ---- CSA and HCA attention at the per-sequence positions
    q = torch.randn(B, Nq, Hh, d, generator=gen).to(tdt)
    Kc = torch.randn(B, N, d, generator=gen).to(tdt)
    Vc = torch.randn(B, N, d, generator=gen).to(tdt)
    Kh = torch.randn(B, N_h, d, generator=gen).to(tdt)
    Vh = torch.randn(B, N_h, d, generator=gen).to(tdt)
    Kr = torch.randn(B, T_raw, d, device=gpu).to(tdt)    # raw rows: position t at row t
    Vr = torch.randn(B, T_raw, d, device=gpu).to(tdt)
    qt, Kct, Vct, Kht, Vht = (t.to(gpu) for t in (q, Kc, Vc, Kh, Vh))
    out_c = torch.full((B, Nq, Hh, d), float("nan"), device=gpu)
    lse_c = torch.full((B, Nq, Hh), float("nan"), device=gpu)
    out_h = torch.full_like(out_c, float("nan"))
    lse_h = torch.full_like(lse_c, float("nan"))
    H.csa_sparse_attn(qt, Kct, Vct, N, idx, Kr, Vr, 0, n_win, 4, 0, scale, out_c, lse_c,
                      seq_pos=seq_pos)
    H.hca_dense_attn(qt, Kht, Vht, N_h, 128, 0, scale, out_h, lse_h, seq_pos=seq_pos)
    torch.cuda.synchronize()
    goc, glc, goh, glh = f64(out_c), f64(lse_c), f64(out_h), f64(lse_h)
    q64, Kc64, Vc64, Kh64, Vh64 = (f64(t) for t in (q, Kc, Vc, Kh, Vh))
    gidx = idx.cpu().numpy().astype(np.int64)
    for b in range(B):
        lo = max(0, pos[b] - n_win - 2)                # the window rows the oracle needs
        hi = pos[b] + Nq
        Kr64, Vr64 = f64(Kr[b, lo:hi]), f64(Vr[b, lo:hi])
        for i in sorted({0, Nq // 2, Nq - 1}):
            p = pos[b] + i
            ro, rl = O.csa_attention(q64[b, i], Kc64[b], Vc64[b], gidx[b, i], Kr64, Vr64, lo, p,
                                     n_win, scale, 4)
            assert_attention_close(goc[b, i], glc[b, i], ro, rl, case["dt"] == "f32",
                                   f"ragged csa seq {b} row {i}")
            ro, rl = O.hca_attention(q64[b, i], Kh64[b], Vh64[b], p, scale, 128)
            assert_attention_close(goh[b, i], glh[b, i], ro, rl, case["dt"] == "f32",
                                   f"ragged hca seq {b} row {i}")
