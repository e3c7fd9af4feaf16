"""Helpers shared by the GPU parity tests: conversions, tolerances, reporting."""
import numpy as np
import torch

import oracle as O


def f64(t):
    """Exact float64 copy of a tensor (bf16 and fp32 widen exactly)."""
    return t.detach().to("cpu", torch.float32).double().numpy()


def dev(a, dtype, device):
    """float64 array holding values of `dtype` -> device tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


def bf16_ulp(x):
    """Distance to the next bf16 above |x| (for |x| in the normal range)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.maximum(x, 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def assert_bf16_within_one_ulp(gpu, ref, what, acc_err=0.0):
    """gpu and ref hold bf16 values; allow adjacent values (double rounding through fp32
    on the GPU vs one rounding from the exact value in the oracle), plus `acc_err`, the
    bound of the GPU's fp32 accumulation error before its final rounding."""
    diff = np.abs(gpu - ref)
    tol = np.maximum(bf16_ulp(ref), bf16_ulp(gpu)) + acc_err
    bad = diff > tol * (1 + 1e-12)
    assert not bad.any(), f"{what}: {bad.sum()} values beyond 1 bf16 ulp, worst {diff.max()}"
    return int((diff > 0).sum())


def assert_attention_close(out, lse, ref_o, ref_l, fp32, what):
    """fp32 inputs: max-abs 1e-4 on the output; bf16 inputs: per (row, head) relative
    max-norm error 2e-2 (|do|_inf / max(|o_ref|_inf, 1e-6)); lse within 1e-3 (abs)."""
    out = np.asarray(out)
    ref_o = np.asarray(ref_o)
    assert out.shape == ref_o.shape, (out.shape, ref_o.shape)
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty-key rows differ"
    assert (out[empty] == 0).all(), f"{what}: empty rows must be zero"
    if fp32:
        err = np.abs(out - ref_o).max() if out.size else 0.0
        assert err <= 1e-4, f"{what}: max-abs error {err}"
    else:
        num = np.abs(out - ref_o).max(axis=-1)
        den = np.maximum(np.abs(ref_o).max(axis=-1), 1e-6)
        rel = (num / den)[~empty] if (~empty).any() else np.zeros(1)
        assert rel.max() <= 2e-2, f"{what}: worst row relative error {rel.max()}"
    le = np.abs(lse[~empty] - ref_l[~empty])
    assert (le <= 1e-3).all(), f"{what}: lse error {le.max()}"


def topk_set_ok(gpu_idx, ref_idx, ref_scores, k, what, rel=1e-5, tol_abs=None):
    """End-to-end index check when scores differ by rounding: the two selections may
    differ only among entries whose exact scores lie within `rel` of the k-th score (or,
    with tol_abs, an array of per-entry absolute tolerances, within tol_abs[j] of it)."""
    g = set(int(j) for j in gpu_idx if j >= 0)
    r = set(int(j) for j in ref_idx if j >= 0)
    assert list(gpu_idx) == sorted(gpu_idx[gpu_idx >= 0]) + [-1] * int((gpu_idx < 0).sum()), \
        f"{what}: not ascending / padded"
    assert len(g) == len(r), f"{what}: sizes differ"
    if g == r:
        return 0
    kth = np.sort(ref_scores)[::-1][min(k, len(ref_scores)) - 1]
    for j in g ^ r:
        tol = rel * max(abs(kth), 1e-30) + 1e-30 if tol_abs is None else tol_abs[j]
        assert abs(ref_scores[j] - kth) <= tol, \
            f"{what}: entry {j} differs away from the threshold ({ref_scores[j]} vs {kth})"
    return len(g ^ r) // 2


def pv_rounding_bound(q, K, V, scale):
    """Bound on the difference between two split plans of the same bf16 16 x 128 attention:
    the P.V product takes the probabilities as bf16, each split rounding them relative to
    its own running maximum (relative error <= 2^-9 per term on each side), so
    |do| <= 2^-8 sum_j p_j |v_j| / sum_j p_j (+ fp32 slack).  q [H, d], K, V [L, d] (float64)."""
    if K.shape[0] == 0:
        return np.full(q.shape, 1e-6)
    w = O.softmax_weights(q, K, scale)
    return 2.0 ** -8 * (w @ np.abs(V)) + 1e-6
