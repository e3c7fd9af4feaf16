"""MXFP4 indexer keys scanned on FP8 operands (the e2m1 codes widened to e4m3, the same e8m0
block scales): every e2m1 value is exact in e4m3, so scores and selection equal the FP4-operand
scan bit for bit, and both match the oracle's exact scores."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import assert_bf16_within_one_ulp, dev, f64

pytestmark = pytest.mark.gpu

CASES = [
    # decode rows (one query per sequence), the workload's head count and width
    dict(B=3, Nq=1, N=20000, H_I=4, d_I=64, k=512, qdt="bf16", sdt="bf16", paged=False),
    # one 32-channel block per key (the second block of every MFMA step is empty)
    dict(B=1, Nq=3, N=1500, H_I=1, d_I=32, k=64, qdt="f32", sdt="f32", paged=False),
    # two MFMA steps per key; 8 heads (both lane halves of the head rows)
    dict(B=2, Nq=2, N=3000, H_I=8, d_I=128, k=100, qdt="bf16", sdt="f32", paged=False),
    dict(B=1, Nq=1, N=2500, H_I=16, d_I=64, k=200, qdt="f32", sdt="bf16", paged=False),
    dict(B=1, Nq=2, N=999, H_I=2, d_I=64, k=64, qdt="bf16", sdt="bf16", paged=False),
    # keys in 128-token pages (32 rows per page) through a block table
    dict(B=2, Nq=1, N=8192, H_I=4, d_I=64, k=256, qdt="bf16", sdt="bf16", paged=True),
]


@pytest.fixture(scope="module")
def H(gpu):
    from long_context_attention_26_amd import hcsa
    return hcsa


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c['B']}-Nq{c['Nq']}-N{c['N']}-"
                         f"H{c['H_I']}-d{c['d_I']}-{c['qdt']}-{c['sdt']}-p{int(c['paged'])}")
def test_mx_fp8_operands(H, gpu, case):
    print(f"mx fp8 {case}", flush=True)
    B, Nq, N, H_I, d_I, k = case["B"], case["Nq"], case["N"], case["H_I"], case["d_I"], case["k"]
    ratio, pos0 = 4, 4 * N - Nq
    rng = np.random.default_rng(31)
    q = O.round_to(rng.standard_normal((B, Nq, H_I, d_I)), case["qdt"])
    w = O.round_fp32(rng.standard_normal((B, Nq, H_I)))      # signed weights
    keys = rng.standard_normal((B, N, d_I))
    codes, se = O.mxfp4_quantize(keys)
    kt = torch.from_numpy(O.mxfp4_pack(codes)).to(gpu)
    kst = torch.from_numpy((se + 127).astype(np.uint8)).to(gpu)
    qt = dev(q, W.torch_dtype(case["qdt"]), gpu)
    wt = dev(w, torch.float32, gpu)
    sdt = H.BF16 if case["sdt"] == "bf16" else H.F32
    sdtype = W.torch_dtype(case["sdt"])

    table = None
    kx, ks = kt, kst
    if case["paged"]:
        nblk = N // 32                                   # 32 indexer keys per 128-token page
        P = B * nblk + 3
        perm = torch.from_numpy(rng.permutation(P)[: B * nblk].astype(np.int32))
        table = perm.view(B, nblk).to(gpu)
        kx = torch.zeros(P, 32, d_I // 2, dtype=torch.uint8, device=gpu)
        ks = torch.zeros(P, 32, d_I // 32, dtype=torch.uint8, device=gpu)
        kx[table.reshape(-1).long()] = kt.reshape(B * nblk, 32, d_I // 2)
        ks[table.reshape(-1).long()] = kst.reshape(B * nblk, 32, d_I // 32)

    def run(fp8, paged):
        sc = torch.zeros(B * Nq, N, device=gpu, dtype=sdtype)
        ix = torch.full((B, Nq, k), -7, dtype=torch.int32, device=gpu)
        H.csa_index_topk(qt, wt, kx if paged else kt, N, ratio, pos0, k, sdt, ix,
                         k_scales=ks if paged else kst, scores_out=sc, mx_fp8=fp8,
                         block_table=table if paged else None)
        torch.cuda.synchronize()
        return sc, ix

    s4, i4 = run(False, False)
    s8, i8 = run(True, False)
    assert torch.equal(s4, s8), "FP8-operand scores differ from the FP4-operand scores"
    assert torch.equal(i4, i8)
    if case["paged"]:
        sp, ip = run(True, True)
        assert torch.equal(sp, s8) and torch.equal(ip, i8), "paged FP8 scan differs"

    # against the oracle: exact scores of the MXFP4 values the kernels see
    keys_seen = O.mxfp4_dequantize(codes, se)
    q_seen = O.mxfp4_roundtrip(q)
    gs = f64(s8)
    gi = i8.cpu().numpy().reshape(B * Nq, k)
    for b in range(B):
        for i in range(Nq):
            r = b * Nq + i
            nv = O.visible_entries(pos0 + i, N, ratio)
            exact = O.index_scores(q_seen[b, i], w[b, i], keys_seen[b], nv, "f32")
            mag = (np.abs(keys_seen[b, :nv]) @ np.abs(q_seen[b, i]).T) @ np.abs(w[b, i])
            acc_err = (d_I + H_I + 4) * 2.0 ** -24 * mag + 1e-30
            if case["sdt"] == "f32":
                assert (np.abs(gs[r, :nv] - exact) <= acc_err).all()
            else:
                assert_bf16_within_one_ulp(gs[r, :nv], O.round_bf16(exact), "bf16 scores", acc_err)
            assert np.array_equal(gi[r], O.select_topk(gs[r], nv, k)), r
