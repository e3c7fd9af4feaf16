"""The four-launch decode step (hcsa_decode_step) on the serving layouts -- caches in 128-token
pages through a block table, raw tokens in a ring, per-sequence positions -- against the same
step as two calls (hcsa_csa_pool_index_topk, then hcsa_csa_hca_attn) on the same layout:
pooled caches and selection equal bit for bit, attention within the bound that the two split
plans' bf16 probabilities allow.  The two-call path on these layouts is tied to the
contiguous one, and that one to the oracle, in the paged, ring and ragged tests; one row here
is also checked against the oracle directly."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import assert_attention_close, f64, pv_rounding_bound

pytestmark = pytest.mark.gpu

P_TOK = 128
RING = 256

CASES = [
    # one position for all sequences: the step completes a 4-token and a 128-token block,
    # pooled from the ring into pages
    dict(name="paged-ring-pool", paged=True, ring=True, pos=[128 * 150 + 127] * 3),
    # per-sequence positions, contiguous caches, nothing to pool
    dict(name="ragged", paged=False, ring=False, pos=[128 * 150 + 127, 9000, 15001]),
    # both
    dict(name="paged-ragged", paged=True, ring=False, pos=[128 * 159 + 5, 4097, 12345]),
    # bf16 indexer keys (the score-array form of the step)
    dict(name="bf16-keys-paged-ring-pool", paged=True, ring=True, pos=[128 * 150 + 127] * 3,
         keys="bf16"),
    dict(name="bf16-keys-paged-ragged", paged=True, ring=False, pos=[128 * 159 + 5, 4097, 12345],
         keys="bf16"),
]


@pytest.fixture(scope="module")
def H(gpu):
    from long_context_attention_26_amd import hcsa
    return hcsa


def _to_pages(x, table, per, P):
    B, nblk = table.shape
    pool = torch.zeros((P, per) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
    pool[table.reshape(-1).long()] = x[:, : nblk * per].reshape((B * nblk, per) + tuple(x.shape[2:]))
    return pool


def _from_pages(pool, table, per):
    B, nblk = table.shape
    return pool[table.reshape(-1).long()].reshape((B, nblk * per) + tuple(pool.shape[2:]))


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_decode_step_layouts(H, gpu, case):
    print(f"decode step layout {case['name']}", flush=True)
    pos = case["pos"]
    B, d, Hh, H_I, d_I, k, w = len(pos), 128, 16, 4, 64, 256, 128
    T = 128 * 160
    N, N_h = T // 4, T // 128
    scale = 1 / math.sqrt(d)
    bf = torch.bfloat16
    g = torch.Generator().manual_seed(29)
    K = torch.randn(B, T, d, generator=g).to(bf).to(gpu)
    V = torch.randn(B, T, d, generator=g).to(bf).to(gpu)
    I = torch.randn(B, T, d_I, generator=g).to(bf).to(gpu)
    om = {n: (torch.randn(r, generator=g) / math.sqrt(r)).to(gpu)
          for n, r in (("ck", 4), ("cv", 4), ("ik", 4), ("hk", 128), ("hv", 128))}
    ragged = len(set(pos)) > 1

    # reference caches: every block pooled from the contiguous raw tokens
    mx = case.get("keys", "mxfp4") == "mxfp4"
    ref = dict(Kc=torch.empty(B, N, d, dtype=bf, device=gpu),
               Vc=torch.empty(B, N, d, dtype=bf, device=gpu),
               Ic=(torch.empty(B, N, d_I // 2, dtype=torch.uint8, device=gpu) if mx
                   else torch.empty(B, N, d_I, dtype=bf, device=gpu)),
               Kh=torch.empty(B, N_h, d, dtype=bf, device=gpu),
               Vh=torch.empty(B, N_h, d, dtype=bf, device=gpu))
    if mx:
        ref["Ics"] = torch.empty(B, N, d_I // 32, dtype=torch.uint8, device=gpu)
    H.compress_kv_batched([H.pool_job(K, om["ck"], 4, ref["Kc"]), H.pool_job(V, om["cv"], 4, ref["Vc"]),
                           H.pool_job(I, om["ik"], 4, ref["Ic"], ref.get("Ics")),
                           H.pool_job(K, om["hk"], 128, ref["Kh"]),
                           H.pool_job(V, om["hv"], 128, ref["Vh"])], B)

    # the step's own blocks (uniform position only) hold junk until the step pools them
    p = pos[0]
    start = {n: t.clone() for n, t in ref.items()}
    if not ragged:
        assert (p + 1) % 128 == 0
        for n, t in start.items():
            j = p // (4 if t.shape[1] == N else 128)
            t.view(torch.uint8)[:, j] = 0x7F

    table, P = None, 0
    if case["paged"]:
        nblk = T // P_TOK
        P = B * nblk + 5
        table = torch.randperm(P, generator=g)[: B * nblk].to(torch.int32).view(B, nblk).to(gpu)

    def layout(c):
        if not case["paged"]:
            return {n: t.clone() for n, t in c.items()}
        return {n: _to_pages(t, table, 32 if t.shape[1] == N else 1, P) for n, t in c.items()}

    # raw tokens: a ring of the last RING positions (raw_pos0 = 0, row = position % RING)
    if case["ring"]:
        Kr = torch.zeros(B, RING, d, dtype=bf, device=gpu)
        Vr, Ir = torch.zeros_like(Kr), torch.zeros(B, RING, d_I, dtype=bf, device=gpu)
        rows = torch.arange(p - RING + 1, p + 1, device=gpu)
        Kr[:, rows % RING], Vr[:, rows % RING], Ir[:, rows % RING] = K[:, rows], V[:, rows], I[:, rows]
        raw_k, raw_v, raw_i, ring = Kr, Vr, Ir, RING
    elif case["paged"]:                  # raw tokens in the pages of the same table
        raw_k, raw_v, raw_i = (_to_pages(x, table, P_TOK, P) for x in (K, V, I))
        ring = 0
    else:
        raw_k, raw_v, raw_i, ring = K, V, I, 0

    def jobs(c):
        if ragged:
            return []
        out = []
        for name, x, o, r in (("Kc", raw_k, "ck", 4), ("Vc", raw_v, "cv", 4), ("Ic", raw_i, "ik", 4),
                              ("Kh", raw_k, "hk", 128), ("Vh", raw_v, "hv", 128)):
            j = p // r
            ys = None
            if name == "Ic" and mx:
                ys = c["Ics"] if case["paged"] else c["Ics"][:, j:j + 1]
            y = c[name] if case["paged"] else c[name][:, j:j + 1]
            out.append(H.pool_job(x, om[o], r, y, ys, T=r, pos0=j * r))
        return out

    qi = torch.randn(B, 1, H_I, d_I, generator=g).to(bf).to(gpu)
    wi = (torch.rand(B, 1, H_I, generator=g) + 0.1).to(gpu)
    q = torch.randn(B, 1, Hh, d, generator=g).to(bf).to(gpu)
    sp = torch.tensor(pos, dtype=torch.int64, device=gpu) if ragged else None
    pos0 = 0 if ragged else p

    def outs():
        return (torch.full((B, 1, Hh, d), float("nan"), device=gpu),
                torch.full((B, 1, Hh), float("nan"), device=gpu),
                torch.full((B, 1, Hh, d), float("nan"), device=gpu),
                torch.full((B, 1, Hh), float("nan"), device=gpu))

    # ---- the four-launch step
    c1 = layout(start)
    idx1 = torch.full((B, 1, k), -7, dtype=torch.int32, device=gpu)
    o1 = outs()
    H.decode_step(jobs(c1), qi, wi, c1["Ic"], H.BF16, idx1, q, c1["Kc"], c1["Vc"], N, k, raw_k,
                  raw_v, 0, w, 4, c1["Kh"], c1["Vh"], N_h, 128, pos0, scale, *o1,
                  k_scales=c1.get("Ics"), seq_pos=sp, block_table=table, raw_ring=ring)
    # ---- the same step as two calls
    c2 = layout(start)
    idx2 = torch.full((B, 1, k), -9, dtype=torch.int32, device=gpu)
    o2 = outs()
    H.csa_pool_index_topk(jobs(c2), qi, wi, c2["Ic"], N, 4, pos0, k, H.BF16, idx2,
                          k_scales=c2.get("Ics"), seq_pos=sp, block_table=table, raw_ring=ring)
    H.csa_hca_attn(q, c2["Kc"], c2["Vc"], N, idx2, raw_k, raw_v, 0, w, 4, c2["Kh"], c2["Vh"], N_h,
                   128, pos0, scale, *o2, seq_pos=sp, block_table=table, raw_ring=ring)
    torch.cuda.synchronize()

    for n in ref:
        assert torch.equal(c1[n], c2[n]), f"{case['name']}: cache {n} differs"
        if case["paged"]:
            per = 32 if ref[n].shape[1] == N else 1
            have = _from_pages(c1[n], table, per)[:, : ref[n].shape[1]]
        else:
            have = c1[n]
        assert torch.equal(have, ref[n]), f"{case['name']}: cache {n} differs from the reference"
    assert torch.equal(idx1, idx2), f"{case['name']}: idx differs"

    qq = f64(q)
    Kc, Vc, Kh, Vh = (f64(ref[n]) for n in ("Kc", "Vc", "Kh", "Vh"))
    Kf, Vf = f64(K), f64(V)
    gi = idx1.cpu().numpy().astype(np.int64)
    for which, (a, la, b, lb) in (("csa", (o1[0], o1[1], o2[0], o2[1])),
                                  ("hca", (o1[2], o1[3], o2[2], o2[3]))):
        a, b, la, lb = f64(a), f64(b), f64(la), f64(lb)
        assert np.array_equal(np.isfinite(la), np.isfinite(lb)), f"{case['name']}: {which} rows"
        fin = np.isfinite(la)
        assert np.abs(la[fin] - lb[fin]).max(initial=0.0) <= 1e-5, f"{case['name']}: {which} lse"
        for bb in range(B):
            pb = pos[bb]
            if which == "csa":
                keys, vals = O.csa_keys(Kc[bb], Vc[bb], gi[bb, 0], Kf[bb], Vf[bb], 0, pb, w,
                                        O.visible_entries(pb, N, 4))
            else:
                n = O.visible_entries(pb, N_h, 128)
                keys, vals = Kh[bb, :n], Vh[bb, :n]
            bound = pv_rounding_bound(qq[bb, 0], keys, vals, scale)
            err = np.abs(a[bb, 0] - b[bb, 0])
            assert (err <= bound).all(), \
                f"{case['name']}: {which} sequence {bb}, worst {(err / bound).max()}"
    # one sequence against the oracle, on the GPU's selection
    bb = B - 1
    pb = pos[bb]
    ro, rl = O.csa_attention(qq[bb, 0], Kc[bb], Vc[bb], gi[bb, 0], Kf[bb], Vf[bb], 0, pb, w,
                             scale, 4)
    assert_attention_close(f64(o1[0][bb, 0]), f64(o1[1][bb, 0]), ro, rl, False,
                           f"{case['name']} csa")
    ro, rl = O.hca_attention(qq[bb, 0], Kh[bb], Vh[bb], pb, scale, 128)
    assert_attention_close(f64(o1[2][bb, 0]), f64(o1[3][bb, 0]), ro, rl, False,
                           f"{case['name']} hca")
