"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, library routines (torch SDPA, numpy/torch casts), brute force on tiny
inputs, hand-derived values and the pages' constants."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


# ----------------------------------------------------------------------- rounding

def test_round_bf16_hand_values():
    one = 1.0
    cases = [
        (one + 2 ** -8, 1.0),                      # tie -> even (mantissa 0)
        (one + 3 * 2 ** -8, one + 2 ** -6),        # tie -> even (mantissa 2)
        (one + 2 ** -8 + 2 ** -30, one + 2 ** -7), # above the tie
        (3.0, 3.0),
        (-(one + 2 ** -8), -1.0),
        ((2 - 2 ** -7) * 2.0 ** 127, (2 - 2 ** -7) * 2.0 ** 127),   # max finite bf16
        ((2 - 2 ** -8) * 2.0 ** 127, math.inf),    # tie at the top rounds to overflow
        (2.0 ** -133, 2.0 ** -133),                # smallest subnormal
        (2.0 ** -134, 0.0),                        # half of it: tie -> even (0)
        (3 * 2.0 ** -134, 2.0 ** -132),            # 1.5 quanta: tie -> even (2 quanta)
        (0.0, 0.0),
    ]
    for x, want in cases:
        assert O.round_bf16(x) == want, (x, O.round_bf16(x), want)


def test_round_bf16_matches_torch_cast():
    x32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-40, 40, 200000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x32.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_fp32_matches_numpy_cast():
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))
    x = np.concatenate([x, [2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -151, 1 + 2.0 ** -24]])
    want = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(O.round_fp32(x), want)


# ----------------------------------------------------------------------- MXFP4

def _e2m1_from_bitfields(code):
    """Value of an FP4 E2M1 code from its bit fields: sign, 2-bit exponent (bias 1),
    1-bit mantissa; exponent field 0 is subnormal (0.5 * m)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m)
    return -mag if s else mag


def test_e2m1_grid_from_bit_fields_and_golden_table():
    with open(os.path.join(GOLDEN, "e2m1_table.json")) as f:
        table = json.load(f)
    for code in range(16):
        v = _e2m1_from_bitfields(code)
        assert v == table["codes"][str(code)]
        assert O.mxfp4_dequantize(np.array([[code] * 32]), np.array([[0]]))[0, 0] == v
    assert O.E2M1_GRID.max() == 2.0 ** table["e2m1_emax"] * 1.5


def test_mxfp4_hand_block():
    # amax = 6 -> floor(log2 6) = 2 -> scale exponent 0; elements are the values themselves
    vals = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 0.1, 2.9, 4.9, -6.0, 0.0,
            0.5]
    want = [7, 0, 2, 2, 4, 4, 6, 6, 8, 14, 0, 5, 6, 15, 0, 1]
    block = np.zeros(32)
    block[: len(vals)] = vals
    codes, se = O.mxfp4_quantize(block[None])
    assert se[0, 0] == 0
    assert list(codes[0, : len(vals)]) == want
    # amax = 7: same exponent, 7 saturates to 6
    codes, se = O.mxfp4_quantize(np.array([[7.0] + [0.0] * 31]))
    assert se[0, 0] == 0 and codes[0, 0] == 7
    # amax = 1 -> exponent -2, so 1.0 is stored as 4 * 2^-2 (code 6); 0.3 / 0.25 = 1.2 -> 1.0
    codes, se = O.mxfp4_quantize(np.array([[1.0, 0.3, -0.125] + [0.0] * 29]))
    assert se[0, 0] == -2 and list(codes[0, :3]) == [6, 2, 8 | 1]
    # amax = 0 -> exponent -127 and all-zero codes
    codes, se = O.mxfp4_quantize(np.zeros((1, 32)))
    assert se[0, 0] == -127 and not codes.any()
    # amax = 2^100 -> exponent 98
    codes, se = O.mxfp4_quantize(np.array([[2.0 ** 100] + [0.0] * 31]))
    assert se[0, 0] == 98 and codes[0, 0] == 6


def test_mxfp4_roundtrip_of_representable_blocks():
    codes = rng.integers(0, 16, size=(500, 64))
    codes[:, 0] = rng.choice([6, 7, 14, 15], size=500)      # fixes the block amax binade
    codes[:, 32] = rng.choice([6, 7, 14, 15], size=500)
    exps = rng.integers(-20, 20, size=(500, 2))
    vals = O.mxfp4_dequantize(codes, exps)
    c2, e2 = O.mxfp4_quantize(vals)
    assert np.array_equal(e2, exps)
    # -0 and +0 both decode to 0; compare decoded values
    assert np.array_equal(O.mxfp4_dequantize(c2, e2), vals)


def test_mxfp4_exhaustive_bf16_inputs_error_bound():
    """Every finite bf16 value v, placed in a block whose amax is 6 * 2^e, decodes to a
    point of the grid within half a grid step of v (or saturates), and the scale
    exponent is e."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    v32 = (bits << 16).view(np.float32)
    v = v32[np.isfinite(v32)].astype(np.float64)
    for e in (-3, 0, 5):
        anchor = 6.0 * 2.0 ** e
        vv = v[np.abs(v) <= anchor]
        pad = (-vv.size) % 31
        body = np.concatenate([vv, np.zeros(pad)]).reshape(-1, 31)
        blocks = np.concatenate([np.full((body.shape[0], 1), anchor), body], axis=1)
        codes, se = O.mxfp4_quantize(blocks)
        assert (se == e).all()
        dq = O.mxfp4_dequantize(codes, se)[:, 1:]
        # half-step bound of the e2m1 grid: 0.25 below 2, 0.5 in [2, 4], 1 in [4, 6]
        a = np.abs(body) / 2.0 ** e
        half = np.where(a <= 2, 0.25, np.where(a <= 4, 0.5, 1.0)) * 2.0 ** e
        assert (np.abs(dq - body) <= half + 0.0).all()
        assert (np.sign(dq) * np.sign(body) >= 0).all()


# ----------------------------------------------------------------------- compression

def test_compress_zero_logits_is_block_mean():
    x = rng.standard_normal((64, 7))
    for r in (1, 2, 4, 16):
        got = O.compress(x, np.zeros(r), r)
        want = x.reshape(64 // r, r, 7).mean(axis=1)
        assert np.allclose(got, want, rtol=0, atol=1e-14)


def test_compress_ratio_one_is_identity():
    x = rng.standard_normal((13, 5))
    assert np.array_equal(O.compress(x, np.array([0.7]), 1), x)


def test_compress_two_point_closed_form():
    # omega = (0, ln 3): weights 1/4 and 3/4
    x = rng.standard_normal((10, 3))
    got = O.compress(x, np.array([0.0, math.log(3.0)]), 2)
    want = 0.25 * x[0::2] + 0.75 * x[1::2]
    assert np.allclose(got, want, atol=1e-15)


def test_compress_one_hot_limit_and_tail():
    x = rng.standard_normal((4 * 9 + 3, 4))          # 3-token tail is not pooled
    got = O.compress(x, np.array([0.0, 0.0, 60.0, 0.0]), 4)
    assert got.shape == (9, 4)
    assert np.allclose(got, x[2:36:4], atol=1e-24 + 1e-12)


def test_entry_counts_from_pages():
    with open(os.path.join(GOLDEN, "pages_constants.json")) as f:
        pc = json.load(f)
    m, mp = pc["csa_ratio_m"], pc["hca_ratio_m_prime"]
    assert (O.CSA_RATIO, O.HCA_RATIO, O.N_WIN) == (m, mp, pc["n_win"])
    assert (O.TOPK_PRO, O.TOPK_FLASH) == (pc["topk_pro"], pc["topk_flash"])
    assert math.lcm(m, mp) == pc["cache_block_tokens_lcm"]
    expected = {4096: (1024, 32), 131072: (32768, 1024), 1048576: (262144, 8192),
                262144: (65536, 2048)}
    for T, (nc, nh) in expected.items():
        assert O.entry_count(T, m) == nc and O.entry_count(T, mp) == nh
        # the last token of the context sees every entry
        assert O.visible_entries(T - 1, nc, m) == nc and O.visible_entries(T - 1, nh, mp) == nh
    # workloads agree
    for cfg in W.CONFIGS.values():
        assert cfg.N_c == cfg.T // 4 and cfg.N_h == cfg.T // 128
    # chunked prefill: the last chunk token sees the chunk's own completed blocks
    assert O.visible_entries(262144 + 4095, 66560, 4) == 66560
    assert O.visible_entries(262144, 66560, 4) == 65536
    assert O.visible_entries(262144 + 4095, 2080, 128) == 2080
    assert O.visible_entries(262144 + 126, 2080, 128) == 2048
    assert O.visible_entries(262144 + 127, 2080, 128) == 2049


# ----------------------------------------------------------------------- indexer and top-k

def _brute_scores(q, w, K, n):
    out = []
    for j in range(n):
        s = 0.0
        for g in range(q.shape[0]):
            dot = 0.0
            for e in range(q.shape[1]):
                dot += q[g, e] * K[j, e]
            s += w[g] * (dot if dot > 0 else 0.0)
        out.append(s)
    return np.array(out)


def test_index_scores_brute_force():
    q = rng.standard_normal((3, 8))
    w = rng.standard_normal(3)          # signed weights too
    K = rng.standard_normal((20, 8))
    got = O.index_scores(q, w, K, 17, "f32")
    want = _brute_scores(q, w, K, 17)
    assert got.shape == (17,)
    assert np.allclose(got, want, rtol=1e-6, atol=1e-6)
    assert np.array_equal(got, got.astype(np.float32).astype(np.float64))
    gb = O.index_scores(q, w, K, 17, "bf16")
    assert np.array_equal(gb, torch.from_numpy(got.astype(np.float32)).to(torch.bfloat16)
                          .to(torch.float64).numpy())


def test_index_scores_single_head_is_relu_dot():
    q = rng.standard_normal((1, 16))
    K = rng.standard_normal((50, 16))
    got = O.index_scores(q, np.array([1.0]), K, 50, "f32")
    want = np.maximum(K @ q[0], 0).astype(np.float32).astype(np.float64)
    assert np.array_equal(got, want)
    # all-negative dot products give +0 scores
    got = O.index_scores(-np.abs(q), np.array([1.0]), np.abs(K), 50, "f32")
    assert (got == 0).all() and not np.signbit(got).any()


def test_topk_brute_force_and_ties():
    for trial in range(50):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, 48))
        s = rng.integers(-3, 4, size=n).astype(np.float64)      # many ties
        n_vis = int(rng.integers(0, n + 1))
        got = O.select_topk(s, n_vis, k)
        ranked = sorted(range(n_vis), key=lambda j: (-s[j], j))[:k]
        want = sorted(ranked) + [-1] * (k - len(ranked))
        assert list(got) == want


def test_topk_special_rows():
    assert list(O.select_topk(np.zeros(10), 10, 4)) == [0, 1, 2, 3]
    assert list(O.select_topk(np.array([-0.0, 0.0, -0.0, 1.0]), 4, 2)) == [0, 3]
    assert list(O.select_topk(np.array([3.0, 1.0]), 2, 5)) == [0, 1, -1, -1, -1]
    assert list(O.select_topk(np.array([-np.inf, -1.0, -np.inf]), 3, 2)) == [0, 1]


def test_topk_invariant_to_positive_weight_scale():
    q = rng.standard_normal((4, 16))
    w = np.abs(rng.standard_normal(4))
    K = rng.standard_normal((300, 16))
    a = O.select_topk(O.index_scores(q, w, K, 300, "f32"), 300, 20)
    b = O.select_topk(O.index_scores(q, 8.0 * w, K, 300, "f32"), 300, 20)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------- attention

def _sdpa(q, K, V, scale, mask=None):
    """torch's scaled_dot_product_attention in fp64 on the CPU (library routine)."""
    qt = torch.from_numpy(q)[None]              # [1, H, d] as (batch, L, E)
    kt = torch.from_numpy(K)[None].expand(1, *K.shape)
    vt = torch.from_numpy(V)[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=m, scale=scale)[0].numpy()


def test_csa_ratio1_full_topk_no_window_is_standard_attention():
    T, H, d = 37, 3, 16
    x_k = rng.standard_normal((T, d))
    x_v = rng.standard_normal((T, d))
    q = rng.standard_normal((H, d))
    Kc = O.compress(x_k, np.array([0.3]), 1)
    Vc = O.compress(x_v, np.array([-1.0]), 1)
    p = T - 1
    idx = O.select_topk(rng.standard_normal(T), T, T)        # every entry selected
    o, lse = O.csa_attention(q, Kc, Vc, idx, x_k, x_v, 0, p, 0, 0.25, ratio=1)
    assert np.allclose(o, _sdpa(q, x_k, x_v, 0.25), atol=1e-12)
    # lse against the closed form log sum exp
    ref = np.log(np.exp(0.25 * q @ x_k.T).sum(axis=1))
    assert np.allclose(lse, ref, atol=1e-12)


def test_csa_window_double_counts_recent_tokens():
    T, H, d, w = 40, 2, 8, 6
    x_k = rng.standard_normal((T, d))
    x_v = rng.standard_normal((T, d))
    q = rng.standard_normal((H, d))
    idx = np.arange(T)
    o, _ = O.csa_attention(q, x_k, x_v, idx, x_k, x_v, 0, T - 1, w, 0.5, ratio=1)
    mask = np.zeros((H, T))
    mask[:, T - w:] = math.log(2.0)          # the last w tokens appear twice
    assert np.allclose(o, _sdpa(q, x_k, x_v, 0.5, mask), atol=1e-12)


def test_causal_prefill_reduces_to_causal_attention():
    T, H, d = 24, 2, 8
    x_k = rng.standard_normal((T, d))
    x_v = rng.standard_normal((T, d))
    qs = rng.standard_normal((T, H, d))
    outs = []
    for p in range(T):
        o, _ = O.hca_attention(qs[p], x_k, x_v, p, 0.3, ratio=1)
        outs.append(o)
    got = np.stack(outs)                                    # [T, H, d]
    qt = torch.from_numpy(qs).permute(1, 0, 2)              # [H, T, d]
    kt = torch.from_numpy(x_k)[None].expand(H, T, d)
    vt = torch.from_numpy(x_v)[None].expand(H, T, d)
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                            scale=0.3).permute(1, 0, 2).numpy()
    assert np.allclose(got, want, atol=1e-12)


def test_softmax_rows_sum_to_one_and_constant_values():
    q = rng.standard_normal((4, 32)) * 3
    K = rng.standard_normal((100, 32))
    P = O.softmax_weights(q, K, 0.2)
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-12)
    Vc = np.tile(rng.standard_normal(32), (100, 1))
    o, _ = O.attend(q, K, Vc, 0.2)
    assert np.allclose(o, Vc[0][None], atol=1e-12)


def test_csa_all_selected_no_window_equals_hca_on_same_cache():
    N, H, d, r = 50, 4, 16, 4
    Kc = rng.standard_normal((N, d))
    Vc = rng.standard_normal((N, d))
    q = rng.standard_normal((H, d))
    p = N * r - 1
    a = O.csa_attention(q, Kc, Vc, np.arange(N), Kc, Vc, 0, p, 0, 0.3, ratio=r)
    b = O.hca_attention(q, Kc, Vc, p, 0.3, ratio=r)
    assert np.allclose(a[0], b[0], atol=1e-13) and np.allclose(a[1], b[1], atol=1e-13)


def test_lse_merge_of_any_partition_equals_unsplit():
    H, d, L = 3, 8, 57
    q = rng.standard_normal((H, d))
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    o_full, lse_full = O.attend(q, K, V, 0.4)
    cuts = [0, 5, 5, 30, 57]                                # includes an empty part
    parts = [O.attend(q, K[a:b], V[a:b], 0.4) for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = O.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    assert np.allclose(o, o_full, atol=1e-13) and np.allclose(lse, lse_full, atol=1e-13)
    o, lse = O.lse_merge(np.zeros((2, H, d)), np.full((2, H), -np.inf))
    assert (o == 0).all() and np.isneginf(lse).all()


def test_empty_key_list():
    o, lse = O.hca_attention(np.ones((2, 4)), np.ones((3, 4)), np.ones((3, 4)), 10, 1.0)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_decode_query_composition_shapes():
    cfg = W.small(W.CONFIGS[1], T=512, pos0=511, topk=16, n_win=8)
    K, V, I = (t.double().numpy() for t in W.raw_sequence(cfg, 0))
    om = {k: v.double().numpy() for k, v in W.pool_logits(cfg).items()}
    q, qi, wi = (t.double().numpy() for t in W.queries(cfg))
    Kc = O.round_fp32(O.compress(K, om["csa_k"], 4))
    Vc = O.round_fp32(O.compress(V, om["csa_v"], 4))
    Ic = O.round_fp32(O.compress(I, om["idx_k"], 4))
    Kh = O.round_fp32(O.compress(K, om["hca_k"], 128))
    Vh = O.round_fp32(O.compress(V, om["hca_v"], 128))
    r = O.decode_query(q[0, 0], qi[0, 0], wi[0, 0], Kc, Vc, Ic, K, V, 0, Kh, Vh, cfg.pos0,
                       cfg.topk, cfg.n_win, cfg.scale, "f32")
    assert r["idx"].shape == (16,) and (np.diff(r["idx"]) > 0).all()
    assert r["csa"][0].shape == (1, 64) and r["hca"][0].shape == (1, 64)


def _sdpa_lse(q, K, V, scale):
    """torch's scaled-dot-product attention (float64, CPU) of every head of q [H, d] over
    K, V [L, d], and the log-sum-exp of the scaled logits (torch.logsumexp)."""
    qt, Kt, Vt = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)) for a in (q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(qt[None], Kt[None], Vt[None],
                                                         scale=scale)[0]
    lse = torch.logsumexp(scale * (qt @ Kt.T), dim=1)
    return o.numpy(), lse.numpy()


def _loop_scores(qi, wi, Ic, n, dtype):
    """Indexer scores by Python loops: sum_g w_g max(0, sum_e q[g, e] k[j, e]), rounded to
    fp32 by numpy's cast, then to bf16 by torch's cast when asked; -0 read as +0."""
    out = []
    for j in range(n):
        s = 0.0
        for g in range(qi.shape[0]):
            dot = 0.0
            for e in range(qi.shape[1]):
                dot += float(qi[g, e]) * float(Ic[j, e])
            s += float(wi[g]) * max(0.0, dot)
        out.append(s)
    x = np.array(out, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    return x.astype(np.float64) + 0.0


def _sorted_topk(scores, k):
    """k largest by sorted() on (-score, index), ascending, padded with -1."""
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))[:k]
    return sorted(order) + [-1] * (k - min(k, len(scores)))


def _composition_case(seed, Nc=64, Nh=3, T=260, d=16, H=3, H_I=2, d_I=8):
    """Independent random arrays for every input of decode_query (distinct per stream, so a
    swapped or misrouted operand changes the result)."""
    g = np.random.default_rng(seed)
    r = lambda *s: g.standard_normal(s)
    return dict(q=r(H, d), qi=r(H_I, d_I), wi=np.abs(r(H_I)), Kc=r(Nc, d), Vc=r(Nc, d),
                Ic=r(Nc, d_I), K=r(T, d), V=r(T, d), Kh=r(Nh, d), Vh=r(Nh, d))


@pytest.mark.parametrize("score_dtype", ["f32", "bf16"])
def test_decode_query_all_selected_no_window_is_sdpa_lse(score_dtype):
    """Every visible entry selected (k >= n_c), no window: the CSA result is plain softmax
    attention over the visible compressed entries, the HCA result over the visible HCA
    entries (n_h = floor((p+1)/128): 2 of the 3 rows at p = 259), both by torch SDPA."""
    c = _composition_case(1)
    p, scale = 259, 0.37
    n_c, n_h = min(64, (p + 1) // 4), min(3, (p + 1) // 128)
    r = O.decode_query(c["q"], c["qi"], c["wi"], c["Kc"], c["Vc"], c["Ic"], c["K"], c["V"], 0,
                       c["Kh"], c["Vh"], p, 100, 0, scale, score_dtype)
    o, lse = _sdpa_lse(c["q"], c["Kc"][:n_c], c["Vc"][:n_c], scale)
    assert np.allclose(r["csa"][0], o, atol=1e-12) and np.allclose(r["csa"][1], lse, atol=1e-12)
    o, lse = _sdpa_lse(c["q"], c["Kh"][:n_h], c["Vh"][:n_h], scale)
    assert np.allclose(r["hca"][0], o, atol=1e-12) and np.allclose(r["hca"][1], lse, atol=1e-12)
    assert list(r["idx"]) == list(range(n_c)) + [-1] * (100 - n_c)


@pytest.mark.parametrize("score_dtype,raw_pos0", [("f32", 0), ("bf16", 0), ("f32", 37)])
def test_decode_query_selection_and_window_against_brute_force(score_dtype, raw_pos0):
    """k < n_c and a window: scores equal the Python-loop scores, idx the sorted() selection
    on them, and the CSA result SDPA over [selected entries] ++ [raw tokens p-w+1 .. p]
    (raw rows held from raw_pos0 on); the HCA result is unaffected by k and the window."""
    c = _composition_case(2)
    p, scale, k, w = 259, 0.29, 10, 16
    n_c, n_h = min(64, (p + 1) // 4), min(3, (p + 1) // 128)
    K, V = c["K"][raw_pos0:], c["V"][raw_pos0:]
    r = O.decode_query(c["q"], c["qi"], c["wi"], c["Kc"], c["Vc"], c["Ic"], K, V, raw_pos0,
                       c["Kh"], c["Vh"], p, k, w, scale, score_dtype)
    sc = _loop_scores(c["qi"], c["wi"], c["Ic"], n_c, score_dtype)
    assert np.array_equal(r["scores"], sc)
    sel = _sorted_topk(list(sc), k)
    assert list(r["idx"]) == sel
    win = list(range(p - w + 1, p + 1))
    keys = np.concatenate([c["Kc"][sel], c["K"][win]])
    vals = np.concatenate([c["Vc"][sel], c["V"][win]])
    o, lse = _sdpa_lse(c["q"], keys, vals, scale)
    assert np.allclose(r["csa"][0], o, atol=1e-12) and np.allclose(r["csa"][1], lse, atol=1e-12)
    o, lse = _sdpa_lse(c["q"], c["Kh"][:n_h], c["Vh"][:n_h], scale)
    assert np.allclose(r["hca"][0], o, atol=1e-12) and np.allclose(r["hca"][1], lse, atol=1e-12)


def test_decode_query_ties_select_lowest_indices():
    """All-zero indexer weights: every score is +0 and the selection is entries 0..k-1."""
    c = _composition_case(3)
    r = O.decode_query(c["q"], c["qi"], 0.0 * c["wi"], c["Kc"], c["Vc"], c["Ic"], c["K"], c["V"],
                       0, c["Kh"], c["Vh"], 259, 7, 4, 0.5, "bf16")
    assert list(r["idx"]) == list(range(7)) and (r["scores"] == 0).all()
    assert not np.signbit(r["scores"]).any()


# --------------------------------------------------------------------------- backward pins
# The gradients are pinned to central finite differences of the forward functions (which
# the pins above tie to the pages and to closed forms), so a wrong sign, a dropped term or
# a transposed product in the backward fails here.

def _fd_grad(f, x, h=1e-6):
    """Central finite-difference gradient of the scalar f at x (every element)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        g[i] = (f(xp) - f(xm)) / (2 * h)
    return g


def _close(a, b, tol=1e-6):
    assert np.allclose(a, b, rtol=tol, atol=tol), np.abs(a - b).max()


def test_attend_backward_matches_finite_differences():
    r = np.random.default_rng(41)
    H, L, d, scale = 3, 6, 5, 0.37
    q, k, v = r.standard_normal((H, d)), r.standard_normal((L, d)), r.standard_normal((L, d))
    do, dl = r.standard_normal((H, d)), r.standard_normal(H)

    def loss(q_, k_, v_):
        o, lse = O.attend(q_, k_, v_, scale)
        return (do * o).sum() + (dl * lse).sum()
    dq, dk, dv = O.attend_backward(q, k, v, scale, do, dl)
    _close(dq, _fd_grad(lambda x: loss(x, k, v), q))
    _close(dk, _fd_grad(lambda x: loss(q, x, v), k))
    _close(dv, _fd_grad(lambda x: loss(q, k, x), v))
    # without dlse the lse term drops out
    dq0, _, _ = O.attend_backward(q, k, v, scale, do)
    _close(dq0, _fd_grad(lambda x: (do * O.attend(x, k, v, scale)[0]).sum(), q))


def test_attend_backward_closed_forms():
    r = np.random.default_rng(42)
    H, L, d, scale = 4, 7, 6, 0.5
    q, k, v = r.standard_normal((H, d)), r.standard_normal((L, d)), r.standard_normal((L, d))
    do, dl = r.standard_normal((H, d)), r.standard_normal(H)
    # the value gradients sum to the summed output gradient (each head's weights sum to one)
    _, _, dv = O.attend_backward(q, k, v, scale, do, dl)
    _close(dv.sum(axis=0), do.sum(axis=0), 1e-12)
    # identical keys: uniform weights, and only the lse term moves q: dq_h = scale dlse_h k
    kk = np.repeat(k[:1], L, axis=0)
    dq, dk, _ = O.attend_backward(q, kk, v, scale, do, dl)
    _close(dq, scale * dl[:, None] * kk[0][None, :], 1e-12)
    # one key: the output is v whatever q is, so dq = scale dlse k and dv = sum_h dout_h
    dq1, dk1, dv1 = O.attend_backward(q, k[:1], v[:1], scale, do, dl)
    _close(dq1, scale * dl[:, None] * k[0][None, :], 1e-12)
    _close(dv1[0], do.sum(axis=0), 1e-12)
    _close(dk1[0], scale * (dl[:, None] * q).sum(axis=0), 1e-12)


def test_csa_backward_matches_finite_differences():
    r = np.random.default_rng(43)
    H, d, N, scale, w = 2, 4, 6, 0.4, 3
    p, raw_pos0 = 13, 9                      # window positions 11..13 -> raw rows 2..4
    Kc, Vc = r.standard_normal((N, d)), r.standard_normal((N, d))
    Kr, Vr = r.standard_normal((6, d)), r.standard_normal((6, d))
    q, do, dl = r.standard_normal((H, d)), r.standard_normal((H, d)), r.standard_normal(H)
    idx = np.array([0, 2, 3, -1, 5])         # 5 is past n_c(13) = 3: skipped, like the padding

    def loss(q_, Kc_, Vc_, Kr_, Vr_):
        o, lse = O.csa_attention(q_, Kc_, Vc_, idx, Kr_, Vr_, raw_pos0, p, w, scale, 4)
        return (do * o).sum() + (dl * lse).sum()
    dq, dKc, dVc, dKr, dVr = O.csa_attention_backward(q, Kc, Vc, idx, Kr, Vr, raw_pos0, p, w,
                                                      scale, do, dl, 4)
    _close(dq, _fd_grad(lambda x: loss(x, Kc, Vc, Kr, Vr), q))
    _close(dKc, _fd_grad(lambda x: loss(q, x, Vc, Kr, Vr), Kc))
    _close(dVc, _fd_grad(lambda x: loss(q, Kc, x, Kr, Vr), Vc))
    _close(dKr, _fd_grad(lambda x: loss(q, Kc, Vc, x, Vr), Kr))
    _close(dVr, _fd_grad(lambda x: loss(q, Kc, Vc, Kr, x), Vr))
    assert not dKc[1].any() and not dKc[4:].any() and not dKr[[0, 1, 5]].any()


def test_hca_backward_matches_finite_differences():
    r = np.random.default_rng(44)
    H, d, N, scale = 3, 4, 5, 0.3
    Kh, Vh = r.standard_normal((N, d)), r.standard_normal((N, d))
    q, do, dl = r.standard_normal((H, d)), r.standard_normal((H, d)), r.standard_normal(H)
    p = 3 * 128 + 5                          # three entries visible

    def loss(q_, K_, V_):
        o, lse = O.hca_attention(q_, K_, V_, p, scale, 128)
        return (do * o).sum() + (dl * lse).sum()
    dq, dK, dV = O.hca_attention_backward(q, Kh, Vh, p, scale, do, dl, 128)
    _close(dq, _fd_grad(lambda x: loss(x, Kh, Vh), q))
    _close(dK, _fd_grad(lambda x: loss(q, x, Vh), Kh))
    _close(dV, _fd_grad(lambda x: loss(q, Kh, x), Vh))
    assert not dK[3:].any()


def test_compress_backward_matches_finite_differences():
    r = np.random.default_rng(45)
    T, D, ratio = 11, 3, 4                   # two entries and a tail of 3 tokens
    x, om = r.standard_normal((T, D)), r.standard_normal(ratio)
    dy = r.standard_normal((T // ratio, D))
    loss = lambda x_, om_: (dy * O.compress(x_, om_, ratio)).sum()
    dx, dom = O.compress_backward(x, om, ratio, dy)
    _close(dx, _fd_grad(lambda v: loss(v, om), x))
    _close(dom, _fd_grad(lambda v: loss(x, v), om))
    assert not dx[8:].any()
    # the weights sum to one, so shifting every logit changes nothing
    assert abs(dom.sum()) < 1e-12
