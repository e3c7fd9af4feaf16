"""Backward (training) parity: the GPU's gradients of CSA and HCA attention and of the block
pooling against the oracle's (which the CPU pins tie to finite differences of the forward).
The backward takes the forward's output and log-sum-exp; the stage tests hand it the oracle's
own (rounded to fp32), so only the backward's arithmetic is measured: fp32 sums of exact
bf16/fp32 inputs, checked to 2e-5 of each gradient's largest magnitude (1e-2 on the
matrix-core path, whose products take bf16 operands).  One case chains the
GPU forward into the GPU backward, as a training step does."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import dev, f64

pytestmark = pytest.mark.gpu

rng = np.random.default_rng(777)


@pytest.fixture(scope="module")
def H(gpu):
    from long_context_attention_26_amd import hcsa
    return hcsa


def _rel_close(got, ref, tol, what):
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(got - ref).max()
    assert err <= tol * scale, f"{what}: max error {err:.3e} vs scale {scale:.3e}"


def _tdt(dt):
    return torch.float32 if dt == "f32" else torch.bfloat16


def _tol(dt, Hh, d):
    """bf16 with 16 heads x 128 runs on the matrix cores, whose products take dS, P and
    dout rounded to bf16 (2^-9 relative each); every other shape sums in fp32."""
    return 1e-2 if (dt == "bf16" and Hh == 16 and d == 128) else 2e-5


CSA_CASES = [
    dict(dt="f32", H=1, d=64, N=1024, k=64, n_win=128, Nq=1, B=1, pos0=4095, dlse=False),
    # chunked rows: windows of neighbouring queries overlap, selections repeat entries
    dict(dt="bf16", H=16, d=128, N=800, k=256, n_win=128, Nq=8, B=2, pos0=3190, dlse=True),
    # k above the visible count (padding), window clipped at position 0
    dict(dt="bf16", H=4, d=64, N=40, k=64, n_win=128, Nq=3, B=1, pos0=60, dlse=True),
    # fp32 16 x 128 (plain-ALU path); head / channel tilings: 32 x 128, 8 x 256, 64 x 64,
    # 5 heads (rounded up to 16)
    dict(dt="f32", H=16, d=128, N=500, k=200, n_win=128, Nq=4, B=2, pos0=1900, dlse=True),
    dict(dt="f32", H=32, d=128, N=300, k=100, n_win=64, Nq=2, B=1, pos0=1300, dlse=True),
    dict(dt="bf16", H=8, d=256, N=200, k=50, n_win=32, Nq=2, B=2, pos0=900, dlse=False),
    dict(dt="f32", H=64, d=64, N=100, k=30, n_win=16, Nq=1, B=1, pos0=420, dlse=True),
    dict(dt="bf16", H=5, d=96, N=150, k=40, n_win=20, Nq=2, B=1, pos0=640, dlse=True),
    # nothing to attend
    dict(dt="f32", H=2, d=32, N=100, k=0, n_win=0, Nq=1, B=1, pos0=399, dlse=True),
    # many query tokens (window rows key-major): raw rows starting past position 0, and
    # windows clipped at position 0 with padded selections
    dict(dt="bf16", H=16, d=128, N=900, k=128, n_win=128, Nq=300, B=2, pos0=3300, dlse=True),
    dict(dt="bf16", H=16, d=128, N=80, k=64, n_win=64, Nq=200, B=1, pos0=20, dlse=False),
    # the same rows with a null workspace: the window rows' gradients stay query-major
    dict(dt="bf16", H=16, d=128, N=900, k=128, n_win=128, Nq=300, B=2, pos0=3300, dlse=True,
         nows=True),
    # selected entries key-major by 128-entry tile: two 4096-token chunks (the second
    # ragged), ten tiles, the last partial
    dict(dt="bf16", H=16, d=128, N=1200, k=32, n_win=16, Nq=4200, B=1, pos0=500, dlse=True),
    # selections with repeated entries, padding and invisible entries anywhere in the list
    # (each listed position is its own key), no window
    dict(dt="bf16", H=16, d=128, N=300, k=96, n_win=0, Nq=40, B=2, pos0=1000, dlse=True,
         dup=True),
]


@pytest.mark.parametrize("case", CSA_CASES, ids=lambda c: f"{c['dt']}-H{c['H']}-d{c['d']}-"
                         f"k{c['k']}-Nq{c['Nq']}" + ("-nows" if c.get("nows") else ""))
def test_csa_backward(H, gpu, case):
    print(f"csa bwd {case}", flush=True)
    B, Nq, Hh, d, N, k, w = case["B"], case["Nq"], case["H"], case["d"], case["N"], case["k"], case["n_win"]
    pos0, dt, ratio = case["pos0"], case["dt"], 4
    scale = 1 / math.sqrt(d)
    raw_pos0 = max(0, pos0 - w - 3)
    T_raw = pos0 + Nq - raw_pos0 + 2
    q = O.round_to(rng.standard_normal((B, Nq, Hh, d)), dt)
    Kc, Vc = (O.round_to(rng.standard_normal((B, N, d)), dt) for _ in range(2))
    Kr, Vr = (O.round_to(rng.standard_normal((B, T_raw, d)), dt) for _ in range(2))
    idx = np.full((B, Nq, k), -1, dtype=np.int64)
    for b in range(B):
        for i in range(Nq):
            nv = O.visible_entries(pos0 + i, N, ratio)
            if k and case.get("dup"):
                idx[b, i] = rng.integers(-3, nv + 5, size=k)
            elif k:
                idx[b, i] = O.select_topk(rng.standard_normal(N), nv, k)
    dout = O.round_fp32(rng.standard_normal((B, Nq, Hh, d)))
    dlse = O.round_fp32(rng.standard_normal((B, Nq, Hh))) if case["dlse"] else None

    # oracle forward (fp64, rounded to fp32 as the backward's inputs) and gradients
    o_ref = np.zeros((B, Nq, Hh, d))
    l_ref = np.zeros((B, Nq, Hh))
    dq_ref = np.zeros((B, Nq, Hh, d))
    dKc_ref, dVc_ref = np.zeros((B, N, d)), np.zeros((B, N, d))
    dKr_ref, dVr_ref = np.zeros((B, T_raw, d)), np.zeros((B, T_raw, d))
    for b in range(B):
        for i in range(Nq):
            p = pos0 + i
            o_ref[b, i], l_ref[b, i] = O.csa_attention(q[b, i], Kc[b], Vc[b], idx[b, i], Kr[b],
                                                       Vr[b], raw_pos0, p, w, scale, ratio)
            g = O.csa_attention_backward(q[b, i], Kc[b], Vc[b], idx[b, i], Kr[b], Vr[b],
                                         raw_pos0, p, w, scale, dout[b, i],
                                         None if dlse is None else dlse[b, i], ratio)
            dq_ref[b, i] = g[0]
            dKc_ref[b] += g[1]
            dVc_ref[b] += g[2]
            dKr_ref[b] += g[3]
            dVr_ref[b] += g[4]
    tdt = _tdt(dt)
    out_t = dev(O.round_fp32(o_ref), torch.float32, gpu)
    lse_t = dev(O.round_fp32(l_ref), torch.float32, gpu)
    # gradients accumulate onto what the buffers hold: start them from known values
    base = [O.round_fp32(rng.standard_normal(s)) for s in ((B, N, d), (B, N, d),
                                                          (B, T_raw, d), (B, T_raw, d))]
    dKc, dVc, dKr, dVr = (dev(x, torch.float32, gpu) for x in base)
    dq = torch.full((B, Nq, Hh, d), float("nan"), device=gpu)
    H.csa_sparse_attn_bwd(dev(q, tdt, gpu), dev(Kc, tdt, gpu), dev(Vc, tdt, gpu), N,
                          torch.from_numpy(idx.astype(np.int32)).to(gpu), dev(Kr, tdt, gpu),
                          dev(Vr, tdt, gpu), raw_pos0, w, ratio, pos0, scale, out_t, lse_t,
                          dev(dout, torch.float32, gpu), dq, dKc, dVc, dKr, dVr,
                          dlse=None if dlse is None else dev(dlse, torch.float32, gpu),
                          key_major=not case.get("nows", False))
    torch.cuda.synchronize()
    tol = _tol(dt, Hh, d)
    _rel_close(f64(dq), dq_ref, tol, "dq")
    _rel_close(f64(dKc) - base[0], dKc_ref, tol, "dKc")
    _rel_close(f64(dVc) - base[1], dVc_ref, tol, "dVc")
    _rel_close(f64(dKr) - base[2], dKr_ref, tol, "dK_raw")
    _rel_close(f64(dVr) - base[3], dVr_ref, tol, "dV_raw")
    if k == 0 and w == 0:
        assert (f64(dq) == 0).all()


HCA_CASES = [
    dict(dt="f32", H=1, d=64, N=32, Nq=1, B=1, pos0=4095, dlse=True),
    dict(dt="bf16", H=16, d=128, N=300, Nq=16, B=2, pos0=128 * 280, dlse=True),   # causal rows
    dict(dt="bf16", H=16, d=128, N=8, Nq=2, B=1, pos0=100, dlse=False),            # nothing visible
    dict(dt="bf16", H=8, d=64, N=50, Nq=3, B=2, pos0=6399, dlse=False),
    # many query tokens (key-major entry gradients): three 128-token chunks, the last ragged,
    # 45 entries (a partial 16-entry tile), and a tile no token of the chunk sees
    dict(dt="bf16", H=16, d=128, N=45, Nq=300, B=2, pos0=128 * 40 - 150, dlse=True),
    dict(dt="bf16", H=16, d=128, N=45, Nq=300, B=1, pos0=128 * 20, dlse=False),
    # a null workspace: the entries' gradients stay query-major
    dict(dt="bf16", H=16, d=128, N=45, Nq=300, B=2, pos0=128 * 40 - 150, dlse=True, nows=True),
]


@pytest.mark.parametrize("case", HCA_CASES, ids=lambda c: f"{c['dt']}-H{c['H']}-N{c['N']}-Nq{c['Nq']}"
                         + ("-nows" if c.get("nows") else ""))
def test_hca_backward(H, gpu, case):
    print(f"hca bwd {case}", flush=True)
    B, Nq, Hh, d, N, pos0, dt = case["B"], case["Nq"], case["H"], case["d"], case["N"], case["pos0"], case["dt"]
    scale = 1 / math.sqrt(d)
    q = O.round_to(rng.standard_normal((B, Nq, Hh, d)), dt)
    Kh, Vh = (O.round_to(rng.standard_normal((B, N, d)), dt) for _ in range(2))
    dout = O.round_fp32(rng.standard_normal((B, Nq, Hh, d)))
    dlse = O.round_fp32(rng.standard_normal((B, Nq, Hh))) if case["dlse"] else None
    o_ref, l_ref = np.zeros((B, Nq, Hh, d)), np.zeros((B, Nq, Hh))
    dq_ref, dK_ref, dV_ref = np.zeros((B, Nq, Hh, d)), np.zeros((B, N, d)), np.zeros((B, N, d))
    for b in range(B):
        for i in range(Nq):
            p = pos0 + i
            o_ref[b, i], l_ref[b, i] = O.hca_attention(q[b, i], Kh[b], Vh[b], p, scale, 128)
            g = O.hca_attention_backward(q[b, i], Kh[b], Vh[b], p, scale, dout[b, i],
                                         None if dlse is None else dlse[b, i], 128)
            dq_ref[b, i] = g[0]
            dK_ref[b] += g[1]
            dV_ref[b] += g[2]
    tdt = _tdt(dt)
    dK = torch.zeros(B, N, d, device=gpu)
    dV = torch.zeros(B, N, d, device=gpu)
    dq = torch.full((B, Nq, Hh, d), float("nan"), device=gpu)
    # the forward's lse is -inf where nothing is visible: hand it over as such
    H.hca_dense_attn_bwd(dev(q, tdt, gpu), dev(Kh, tdt, gpu), dev(Vh, tdt, gpu), N, 128, pos0,
                         scale, dev(O.round_fp32(o_ref), torch.float32, gpu),
                         dev(l_ref, torch.float32, gpu), dev(dout, torch.float32, gpu), dq, dK,
                         dV, dlse=None if dlse is None else dev(dlse, torch.float32, gpu),
                         key_major=not case.get("nows", False))
    torch.cuda.synchronize()
    tol = _tol(dt, Hh, d)
    _rel_close(f64(dq), dq_ref, tol, "dq")
    _rel_close(f64(dK), dK_ref, tol, "dKh")
    _rel_close(f64(dV), dV_ref, tol, "dVh")


@pytest.mark.parametrize("ratio,T,D,B,io", [(4, 1003, 64, 2, "bf16"), (128, 1000, 128, 1, "f32"),
                                            (4, 4096, 128, 3, "bf16"), (1, 37, 32, 1, "f32")])
def test_compress_backward(H, gpu, ratio, T, D, B, io):
    print(f"pool bwd r{ratio} T{T} D{D} B{B} {io}", flush=True)
    x = O.round_to(rng.standard_normal((B, T, D)), io)
    om = O.round_fp32(rng.standard_normal(ratio) / math.sqrt(ratio))
    n = T // ratio
    dy = O.round_fp32(rng.standard_normal((B, n, D)))
    dx0 = O.round_fp32(rng.standard_normal((B, T, D)))
    dom0 = O.round_fp32(rng.standard_normal(ratio))
    dx_ref = np.zeros((B, T, D))
    dom_ref = np.zeros(ratio)
    gmag = np.zeros(ratio)
    for b in range(B):
        gx, go = O.compress_backward(x[b], om, ratio, dy[b])
        dx_ref[b] = gx
        dom_ref += go
        blocks = x[b, : n * ratio].reshape(n, ratio, D)
        gmag += np.einsum("jid,jd->i", np.abs(blocks), np.abs(dy[b]))
    dx = dev(dx0, torch.float32, gpu)
    dom = dev(dom0, torch.float32, gpu)
    H.compress_kv_bwd(dev(x, _tdt(io), gpu), dev(om, torch.float32, gpu), ratio,
                      dev(dy, torch.float32, gpu), dx, dom)
    torch.cuda.synchronize()
    # dx: one fma of the device's fp32 softmax weight onto the starting value (a few ulp)
    got = f64(dx)
    assert np.abs(got - (dx0 + dx_ref)).max() <= 2.0 ** -20 * (np.abs(dx0) + np.abs(dx_ref)).max()
    assert (got[:, n * ratio:] == dx0[:, n * ratio:]).all()          # the tail is untouched
    # domega: each g_i is a chain of about D + B*n/256 + 16 fp32 additions of products
    # bounded by gmag_i; four times that chain's worst-case rounding bound
    alpha = O.pool_weights(om)
    chain = D + B * n / 256 + 16
    bound = 4 * chain * 2.0 ** -24 * (alpha * gmag + alpha * (alpha * gmag).sum()).max() \
        + 2.0 ** -23 * np.abs(dom0 + dom_ref).max()
    assert np.abs(f64(dom) - (dom0 + dom_ref)).max() <= bound


def test_training_step_chain(H, gpu):
    """GPU forward -> GPU backward for one chunk of CSA and HCA rows, against the oracle's
    gradients (the forward's bf16 rounding of the probabilities enters through out)."""
    B, Nq, Hh, d, N, Nh, k, w = 1, 16, 16, 128, 600, 20, 128, 128
    pos0, scale = 2400, 1 / math.sqrt(128)
    q = O.round_to(rng.standard_normal((B, Nq, Hh, d)), "bf16")
    Kc, Vc = (O.round_to(rng.standard_normal((B, N, d)), "bf16") for _ in range(2))
    Kh, Vh = (O.round_to(rng.standard_normal((B, Nh, d)), "bf16") for _ in range(2))
    Kr, Vr = (O.round_to(rng.standard_normal((B, pos0 + Nq, d)), "bf16") for _ in range(2))
    idx = np.stack([O.select_topk(rng.standard_normal(N), O.visible_entries(pos0 + i, N, 4), k)
                    for i in range(Nq)])[None]
    dout = O.round_fp32(rng.standard_normal((B, Nq, Hh, d)))
    qt, Kct, Vct, Kht, Vht, Krt, Vrt = (dev(t, torch.bfloat16, gpu) for t in (q, Kc, Vc, Kh, Vh, Kr, Vr))
    it = torch.from_numpy(idx.astype(np.int32)).to(gpu)
    dot = dev(dout, torch.float32, gpu)
    oc = torch.empty(B, Nq, Hh, d, device=gpu)
    lc = torch.empty(B, Nq, Hh, device=gpu)
    oh, lh = torch.empty_like(oc), torch.empty_like(lc)
    H.csa_sparse_attn(qt, Kct, Vct, N, it, Krt, Vrt, 0, w, 4, pos0, scale, oc, lc)
    H.hca_dense_attn(qt, Kht, Vht, Nh, 128, pos0, scale, oh, lh)
    dqc, dqh = torch.empty_like(oc), torch.empty_like(oc)
    dKc, dVc = torch.zeros(B, N, d, device=gpu), torch.zeros(B, N, d, device=gpu)
    dKr, dVr = torch.zeros(B, pos0 + Nq, d, device=gpu), torch.zeros(B, pos0 + Nq, d, device=gpu)
    dKh, dVh = torch.zeros(B, Nh, d, device=gpu), torch.zeros(B, Nh, d, device=gpu)
    H.csa_sparse_attn_bwd(qt, Kct, Vct, N, it, Krt, Vrt, 0, w, 4, pos0, scale, oc, lc, dot, dqc,
                          dKc, dVc, dKr, dVr)
    H.hca_dense_attn_bwd(qt, Kht, Vht, Nh, 128, pos0, scale, oh, lh, dot, dqh, dKh, dVh)
    torch.cuda.synchronize()
    ref = {n_: np.zeros(s) for n_, s in (("dqc", (Nq, Hh, d)), ("dKc", (N, d)), ("dVc", (N, d)),
                                         ("dKr", (pos0 + Nq, d)), ("dVr", (pos0 + Nq, d)),
                                         ("dqh", (Nq, Hh, d)), ("dKh", (Nh, d)), ("dVh", (Nh, d)))}
    for i in range(Nq):
        g = O.csa_attention_backward(q[0, i], Kc[0], Vc[0], idx[0, i], Kr[0], Vr[0], 0, pos0 + i,
                                     w, scale, dout[0, i], None, 4)
        ref["dqc"][i] = g[0]
        for n_, x in zip(("dKc", "dVc", "dKr", "dVr"), g[1:]):
            ref[n_] += x
        g = O.hca_attention_backward(q[0, i], Kh[0], Vh[0], pos0 + i, scale, dout[0, i], None, 128)
        ref["dqh"][i] = g[0]
        ref["dKh"] += g[1]
        ref["dVh"] += g[2]
    got = dict(dqc=dqc[0], dKc=dKc[0], dVc=dVc[0], dKr=dKr[0], dVr=dVr[0], dqh=dqh[0],
               dKh=dKh[0], dVh=dVh[0])
    for n_, t in got.items():
        _rel_close(f64(t), ref[n_], 2e-2, n_)


@pytest.mark.parametrize("dt,Hh,d,Nq", [("bf16", 16, 128, 2), ("f32", 4, 64, 2),
                                         ("bf16", 16, 128, 24)])
def test_backward_ragged_positions(H, gpu, dt, Hh, d, Nq):
    """Per-sequence positions (seq_pos): each sequence's gradients against the oracle at its
    own position, CSA and HCA (24 tokens: the key-major passes)."""
    print(f"bwd ragged {dt} H{Hh} d{d} Nq{Nq}", flush=True)
    pos = [5000, 777, 2999]
    B, k, w = len(pos), 128, 64
    scale = 1 / math.sqrt(d)
    top = max(pos) + Nq
    N, Nh = top // 4 + 2, top // 128 + 1
    q = O.round_to(rng.standard_normal((B, Nq, Hh, d)), dt)
    Kc, Vc = (O.round_to(rng.standard_normal((B, N, d)), dt) for _ in range(2))
    Kh, Vh = (O.round_to(rng.standard_normal((B, Nh, d)), dt) for _ in range(2))
    Kr, Vr = (O.round_to(rng.standard_normal((B, top, d)), dt) for _ in range(2))
    idx = np.stack([np.stack([O.select_topk(rng.standard_normal(N),
                                            O.visible_entries(pos[b] + i, N, 4), k)
                              for i in range(Nq)]) for b in range(B)])
    dout = O.round_fp32(rng.standard_normal((B, Nq, Hh, d)))
    dlse = O.round_fp32(rng.standard_normal((B, Nq, Hh)))
    oc, lc, oh, lh = (np.zeros(s) for s in ((B, Nq, Hh, d), (B, Nq, Hh), (B, Nq, Hh, d), (B, Nq, Hh)))
    ref = {n: np.zeros(s) for n, s in (("dqc", (B, Nq, Hh, d)), ("dKc", (B, N, d)), ("dVc", (B, N, d)),
                                      ("dKr", (B, top, d)), ("dVr", (B, top, d)),
                                      ("dqh", (B, Nq, Hh, d)), ("dKh", (B, Nh, d)), ("dVh", (B, Nh, d)))}
    for b in range(B):
        for i in range(Nq):
            p = pos[b] + i
            oc[b, i], lc[b, i] = O.csa_attention(q[b, i], Kc[b], Vc[b], idx[b, i], Kr[b], Vr[b],
                                                 0, p, w, scale, 4)
            oh[b, i], lh[b, i] = O.hca_attention(q[b, i], Kh[b], Vh[b], p, scale, 128)
            g = O.csa_attention_backward(q[b, i], Kc[b], Vc[b], idx[b, i], Kr[b], Vr[b], 0, p, w,
                                         scale, dout[b, i], dlse[b, i], 4)
            ref["dqc"][b, i] = g[0]
            for n_, x in zip(("dKc", "dVc", "dKr", "dVr"), g[1:]):
                ref[n_][b] += x
            g = O.hca_attention_backward(q[b, i], Kh[b], Vh[b], p, scale, dout[b, i],
                                         dlse[b, i], 128)
            ref["dqh"][b, i] = g[0]
            ref["dKh"][b] += g[1]
            ref["dVh"][b] += g[2]
    tdt = _tdt(dt)
    f32 = lambda x: dev(O.round_fp32(x), torch.float32, gpu)
    sp = torch.tensor(pos, dtype=torch.int64, device=gpu)
    qt = dev(q, tdt, gpu)
    got = {n_: torch.zeros(v.shape, device=gpu) for n_, v in ref.items()}
    H.csa_sparse_attn_bwd(qt, dev(Kc, tdt, gpu), dev(Vc, tdt, gpu), N,
                          torch.from_numpy(idx.astype(np.int32)).to(gpu), dev(Kr, tdt, gpu),
                          dev(Vr, tdt, gpu), 0, w, 4, 0, scale, f32(oc), f32(lc), f32(dout),
                          got["dqc"], got["dKc"], got["dVc"], got["dKr"], got["dVr"],
                          dlse=f32(dlse), seq_pos=sp)
    H.hca_dense_attn_bwd(qt, dev(Kh, tdt, gpu), dev(Vh, tdt, gpu), Nh, 128, 0, scale, f32(oh),
                         dev(lh, torch.float32, gpu), f32(dout), got["dqh"], got["dKh"],
                         got["dVh"], dlse=f32(dlse), seq_pos=sp)
    torch.cuda.synchronize()
    tol = _tol(dt, Hh, d)
    for n_, t in got.items():
        _rel_close(f64(t), ref[n_], tol, f"ragged {n_}")
