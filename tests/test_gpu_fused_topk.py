"""Indexer + top-k of MXFP4 keys without the score array (hcsa_csa_index_topk with no
score copy, few long rows, bf16 scores): a floor per row from scored samples, per-chunk
candidate lists from the scan, the exact threshold among the candidates, and a rescan of
rows whose lists hold too few or too many candidates.  The selection must equal that of
the two-call path (scores, then hcsa_topk on them) bit for bit, and the oracle's selection
on those scores; the two-call path is checked against the oracle's scores elsewhere."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H(gpu):
    from long_context_attention_26_amd import hcsa
    return hcsa


def _nv(p, N):
    return min(N, (p + 1) // 4)


CASES = [
    # every row on the list path
    dict(name="b4-262144-k1024", B=4, Nq=1, N=262144, pos=[4 * 262144 - 1] * 4, k=1024, H_I=4,
         d_I=64),
    # ragged positions, f32 queries, 8 heads x 128 channels
    dict(name="ragged-f32q", B=3, Nq=1, N=300000, pos=[4 * 300000 - 1, 4 * 123457 + 2, 4 * 70001],
         k=512, H_I=8, d_I=128, qdt="f32"),
    # rows of <= 4096 visible keys (every key a candidate) and a row seeing fewer than k
    dict(name="short-rows", B=3, Nq=1, N=6000, pos=[4 * 6000 - 1, 4 * 3000 - 1, 4 * 200 - 1],
         k=256, H_I=1, d_I=32),
    # every score 0: the floor admits every key, the row is rescanned; ties to the lowest index
    dict(name="all-ties-rescan", B=2, Nq=1, N=40000, pos=[4 * 40000 - 1, 4 * 39000 - 1], k=700,
         H_I=4, d_I=64, w_zero=True),
    # k near the visible count: almost every key is a candidate
    dict(name="dense-k4096", B=1, Nq=1, N=4300, pos=[4 * 4300 - 1], k=4096, H_I=4, d_I=64),
    # large keys planted at exactly the floor's sample positions (32 runs of 128 keys at
    # r * (nv - 128) // 31): the floor lands above the k-th largest key, the list holds
    # fewer than k candidates and the row is rescanned
    dict(name="sampled-runs-rescan", B=1, Nq=1, N=262144, pos=[4 * 262144 - 1], k=1024, H_I=4,
         d_I=64, boost_samples=True),
    # paged keys on FP8 operands
    dict(name="paged-fp8", B=2, Nq=1, N=70000, pos=[4 * 70000 - 1, 4 * 51234 + 1], k=1024, H_I=4,
         d_I=64, paged=True, fp8=True),
    # several query tokens per sequence (few rows), 16 heads
    dict(name="nq8-h16", B=1, Nq=8, N=100000, pos=[4 * 99990], k=1024, H_I=16, d_I=64),
    # large scales on one stretch: the top keys crowd a few chunks
    dict(name="skewed", B=2, Nq=1, N=200000, pos=[4 * 200000 - 1] * 2, k=1024, H_I=4, d_I=64,
         skew=(50000, 58000)),
    # every score 0 and 15 873 .. 16 384 candidates: the resolve's prefix form puts 32 tied
    # candidates on a thread (its counts need 6 bits); expected 0 .. k-1
    dict(name="all-ties-16000", B=1, Nq=1, N=16000, pos=[4 * 16000 - 1], k=1024, H_I=4,
         d_I=64, w_zero=True, expect_first_k=True),
    dict(name="all-ties-16384", B=1, Nq=1, N=16384, pos=[4 * 16384 - 1], k=1024, H_I=4,
         d_I=64, w_zero=True, expect_first_k=True),
    # zero keys (score 0) except a run of 32 keys scoring above 0 that one resolve thread
    # holds whole: 32 candidates above the threshold on one thread
    dict(name="planted-run-16000", B=1, Nq=1, N=16000, pos=[4 * 16000 - 1], k=1024, H_I=4,
         d_I=64, zero_codes=True, plant=(3200, 3232)),
]


def _page_pool(x, table, per, gpu):
    """x [B, n, ...] into a pool of pages of `per` rows at the table's page numbers."""
    B, nblk = table.shape
    P = int(table.max().item()) + 3
    pool = torch.zeros((P, per) + tuple(x.shape[2:]), dtype=x.dtype, device=gpu)
    full = torch.zeros((B, nblk * per) + tuple(x.shape[2:]), dtype=x.dtype, device=gpu)
    n = min(x.shape[1], nblk * per)
    full[:, :n] = x[:, :n]
    pool[table.reshape(-1).long()] = full.reshape((B * nblk, per) + tuple(x.shape[2:]))
    return pool


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_fused_index_topk_equals_two_calls(H, gpu, case):
    print(f"fused index-topk {case['name']}", flush=True)
    B, Nq, N, k, H_I, d_I = case["B"], case["Nq"], case["N"], case["k"], case["H_I"], case["d_I"]
    g = torch.Generator().manual_seed(77)
    Nt = N + 3
    codes = torch.randint(0, 256, (B, Nt, d_I // 2), generator=g, dtype=torch.uint8)
    scales = torch.randint(120, 128, (B, Nt, d_I // 32), generator=g, dtype=torch.uint8)
    if "skew" in case:
        lo, hi = case["skew"]
        scales[:, lo:hi] = 131
    if case.get("boost_samples"):
        for b in range(B):
            nv = _nv(case["pos"][b], N)
            for run in range(32):
                r0 = run * (nv - 128) // 31
                scales[b, r0:r0 + 128] = 134
    if case.get("zero_codes"):
        codes.zero_()
    if "plant" in case:                 # positive e2m1 codes (magnitudes 1..7 in both nibbles)
        lo, hi = case["plant"]
        mag = torch.randint(1, 8, (B, hi - lo, d_I // 2, 2), generator=g, dtype=torch.uint8)
        codes[:, lo:hi] = mag[..., 0] | (mag[..., 1] << 4)
    qdt = torch.float32 if case.get("qdt") == "f32" else torch.bfloat16
    q = torch.randn(B, Nq, H_I, d_I, generator=g)
    if "plant" in case:                 # positive queries: the planted keys score above 0
        q = q.abs() + 0.25
    q = q.to(qdt).to(gpu)
    w = (torch.randn(B, Nq, H_I, generator=g).abs() / math.sqrt(H_I)).to(gpu)
    if case.get("w_zero"):
        w.zero_()
    seq_pos = torch.tensor(case["pos"], dtype=torch.int64, device=gpu)
    codes, scales = codes.to(gpu), scales.to(gpu)
    table = None
    kc, ks = codes, scales
    if case.get("paged"):
        nblk = -(-Nt // 32)
        perm = torch.randperm(B * nblk + 5, generator=g)[: B * nblk].to(torch.int32)
        table = perm.view(B, nblk).to(gpu)
        kc, ks = _page_pool(codes, table, 32, gpu), _page_pool(scales, table, 32, gpu)
    fp8 = case.get("fp8", False)

    idx = torch.full((B, Nq, k), -7, dtype=torch.int32, device=gpu)
    H.csa_index_topk(q, w, kc, N, 4, 0, k, H.BF16, idx, k_scales=ks, seq_pos=seq_pos,
                     block_table=table, mx_fp8=fp8)
    # a second call on a fresh workspace holding junk: nothing carries over
    ws = H.alloc_workspace(H.index_topk_workspace_size(B, Nq, N, k, H.BF16), gpu)
    ws.fill_(0x5A)
    idx_b = torch.full_like(idx, -7)
    H.csa_index_topk(q, w, kc, N, 4, 0, k, H.BF16, idx_b, k_scales=ks, seq_pos=seq_pos,
                     block_table=table, mx_fp8=fp8, workspace=ws)
    # two calls: scores, then the selector on them
    scores = torch.zeros(B * Nq, N, dtype=torch.bfloat16, device=gpu)
    H.csa_index_scores(q, w, kc, N, 4, 0, scores, k_scales=ks, seq_pos=seq_pos,
                       block_table=table, mx_fp8=fp8)
    idx2 = torch.full_like(idx, -7)
    H.topk(scores, B, Nq, N, 4, 0, k, idx2.view(B * Nq, k), seq_pos=seq_pos)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_b), "fused selection depends on the workspace's contents"
    got, want = idx.view(B * Nq, k).cpu().numpy(), idx2.view(B * Nq, k).cpu().numpy()
    for r in range(B * Nq):
        assert np.array_equal(got[r], want[r]), (case["name"], r)
    if case.get("expect_first_k"):
        assert np.array_equal(got[0], np.arange(k)), case["name"]
    if "plant" in case:
        lo, hi = case["plant"]
        want_p = np.sort(np.concatenate([np.arange(k - (hi - lo)), np.arange(lo, hi)]))
        assert np.array_equal(got[0], want_p), case["name"]
    # the oracle's selection on the GPU's scores, for a few rows
    sc = f64(scores)
    for r in sorted({0, B * Nq - 1}):
        b, i = divmod(r, Nq)
        nv = _nv(case["pos"][b] + i, N)
        assert np.array_equal(got[r], O.select_topk(sc[r], nv, k)), (case["name"], r)


POOL_CASES = [
    # the query token completes a 4-token and a 128-token block
    dict(name="decode-b4", B=4, Nq=1, P=128 * 2188 - 1, k=1024, paged=False, fp8=False),
    dict(name="decode-paged-fp8", B=2, Nq=1, P=128 * 1563 - 1, k=512, paged=True, fp8=True),
    dict(name="nq4", B=2, Nq=4, P=4 * 40000 - 2, k=700, paged=False, fp8=False),
    dict(name="bf16-keys", B=2, Nq=1, P=4 * 30000 - 1, k=512, paged=False, fp8=False,
         bf16_keys=True),
    # raw tokens in a ring of 256 rows per sequence (the state cache)
    dict(name="ring", B=3, Nq=1, P=128 * 700 - 1, k=1024, paged=False, fp8=False, ring=256),
]


@pytest.mark.parametrize("case", POOL_CASES, ids=[c["name"] for c in POOL_CASES])
def test_pool_index_topk_equals_separate_calls(H, gpu, case):
    """Pooling + indexer + top-k in one call against the pooling call then the indexer +
    top-k call: the same pooled caches and the same selection, bit for bit.  The jobs pool
    the blocks the query tokens complete (indexer keys, a 4-token K stream and a 128-token
    K stream); with MXFP4 keys the pooling shares the launch of the selection floors."""
    print(f"pool + index-topk {case['name']}", flush=True)
    B, Nq, P, k = case["B"], case["Nq"], case["P"], case["k"]
    d_I, H_I, D = 64, 4, 128
    T = P + Nq                                    # raw tokens up to the last query
    N = T // 4 + 4
    g = torch.Generator().manual_seed(5)
    Ir = torch.randn(B, T, d_I, generator=g).to(torch.bfloat16).to(gpu)
    Kr = torch.randn(B, T, D, generator=g).to(torch.bfloat16).to(gpu)
    om4 = (torch.randn(4, generator=g) / 2).to(gpu)
    om128 = (torch.randn(128, generator=g) / 11).to(gpu)
    q = torch.randn(B, Nq, H_I, d_I, generator=g).to(torch.bfloat16).to(gpu)
    w = (torch.randn(B, Nq, H_I, generator=g).abs() / 2).to(gpu)
    mx = not case.get("bf16_keys")

    def fresh():
        c = {}
        if mx:
            c["Ic"] = torch.zeros(B, N, d_I // 2, dtype=torch.uint8, device=gpu)
            c["Ics"] = torch.zeros(B, N, d_I // 32, dtype=torch.uint8, device=gpu)
        else:
            c["Ic"], c["Ics"] = torch.zeros(B, N, d_I, dtype=torch.bfloat16, device=gpu), None
        c["Kc"] = torch.zeros(B, N, D, dtype=torch.bfloat16, device=gpu)
        c["Kh"] = torch.zeros(B, N // 32 + 1, D, dtype=torch.bfloat16, device=gpu)
        # entries completed before the first query token
        H.compress_kv_batched([H.pool_job(Ir[:, :P], om4, 4, c["Ic"], c["Ics"]),
                               H.pool_job(Kr[:, :P], om4, 4, c["Kc"]),
                               H.pool_job(Kr[:, :P], om128, 128, c["Kh"])], B)
        return c

    def jobs(c):
        out = []
        for ratio, x, om, y, ys in ((4, Ir, om4, c["Ic"], c["Ics"]), (4, Kr, om4, c["Kc"], None),
                                    (128, Kr, om128, c["Kh"], None)):
            j0, j1 = -(-(P + 1) // ratio) - 1, (P + Nq) // ratio
            if j1 > j0:
                out.append(H.pool_job(x[:, j0 * ratio: j1 * ratio], om, ratio, y[:, j0:j1],
                                      None if ys is None else ys[:, j0:j1]))
        return out

    table = None
    ca, cb = fresh(), fresh()
    if case["paged"]:
        nblk = -(-T // 128)
        perm = torch.randperm(B * nblk + 3, generator=g)[: B * nblk].to(torch.int32)
        table = perm.view(B, nblk).to(gpu)

        def paged(c):
            r = {"Ic": _page_pool(c["Ic"], table, 32, gpu), "Ics": _page_pool(c["Ics"], table, 32, gpu),
                 "Kc": _page_pool(c["Kc"], table, 32, gpu), "Kh": _page_pool(c["Kh"], table, 1, gpu)}
            return r
        ca, cb = paged(ca), paged(cb)
        Irp, Krp = _page_pool(Ir, table, 128, gpu), _page_pool(Kr, table, 128, gpu)

        def jobs(c):                                         # noqa: F811 (paged form)
            out = []
            for ratio, x, om, y, ys in ((4, Irp, om4, c["Ic"], c["Ics"]), (4, Krp, om4, c["Kc"], None),
                                        (128, Krp, om128, c["Kh"], None)):
                j0, j1 = -(-(P + 1) // ratio) - 1, (P + Nq) // ratio
                if j1 > j0:
                    out.append(H.pool_job(x, om, ratio, y, ys, T=(j1 - j0) * ratio,
                                          pos0=j0 * ratio))
            return out
    ring = case.get("ring", 0)
    if ring:
        # the last `ring` raw tokens of each sequence, position t in row t mod ring
        rows = torch.arange(T - ring, T, device=gpu)
        Ir_ring = torch.zeros(B, ring, d_I, dtype=torch.bfloat16, device=gpu)
        Kr_ring = torch.zeros(B, ring, D, dtype=torch.bfloat16, device=gpu)
        Ir_ring[:, rows % ring] = Ir[:, rows]
        Kr_ring[:, rows % ring] = Kr[:, rows]

        def jobs(c):                                         # noqa: F811 (ring form)
            out = []
            for ratio, x, om, y, ys in ((4, Ir_ring, om4, c["Ic"], c["Ics"]),
                                        (4, Kr_ring, om4, c["Kc"], None),
                                        (128, Kr_ring, om128, c["Kh"], None)):
                j0, j1 = -(-(P + 1) // ratio) - 1, (P + Nq) // ratio
                if j1 > j0:
                    out.append(H.pool_job(x, om, ratio, y[:, j0:j1],
                                          None if ys is None else ys[:, j0:j1],
                                          T=(j1 - j0) * ratio, pos0=j0 * ratio))
            return out
    fp8 = case["fp8"]
    idx_a = torch.full((B, Nq, k), -7, dtype=torch.int32, device=gpu)
    idx_b = torch.full_like(idx_a, -7)
    H.compress_kv_batched(jobs(ca), B, block_table=table, raw_ring=ring)
    H.csa_index_topk(q, w, ca["Ic"], N, 4, P, k, H.BF16, idx_a, k_scales=ca["Ics"],
                     block_table=table, mx_fp8=fp8)
    H.csa_pool_index_topk(jobs(cb), q, w, cb["Ic"], N, 4, P, k, H.BF16, idx_b,
                          k_scales=cb["Ics"], block_table=table, raw_ring=ring, mx_fp8=fp8)
    torch.cuda.synchronize()
    for name in ca:
        if ca[name] is not None:
            assert torch.equal(ca[name], cb[name]), f"{case['name']}: pooled {name} differs"
    assert torch.equal(idx_a, idx_b), f"{case['name']}: selection differs"
    assert (idx_a[:, :, 0] >= 0).all()
