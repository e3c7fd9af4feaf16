"""Plain CPU oracle for the hybrid compressed attention (CSA + HCA) of DeepSeek-V4.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  It shares no code with the
HIP library: every function here is written from the method's description, in float64
(numpy), with no blocking, fusion or reordering beyond what the definition states.

Sources (web pages about the DeepSeek-V4 release):
  [LH]   Lighthouse, "deep deepseek v4 release", section 八 (technical report walk-through):
         item 3 "CSA 与 HCA" -- CSA compresses the KV of every m = 4 tokens into one entry,
         a Lightning Indexer picks the top-k compressed entries (k = 1024 Pro / 512 Flash)
         for sparse attention, and a sliding-window branch with n_win = 128 recovers nearby
         tokens; HCA merges every m' = 128 tokens into one entry and keeps dense attention.
         item 7 "异构 KV cache 管理" -- the indexer keeps its own compressed keys; blocks are
         aligned to lcm(m, m').
  [TL]   tulong.co Q&A, "技术架构创新" item 1 -- CSA: every 4 tokens become one block with
         sparse retrieval; HCA: every 128 tokens become one entry.
  [9F]   9fzt.com digest, item 4 (FP4 QAT) -- FP4 on the indexer's QK path; index scores
         are FP32 compressed to BF16 for the top-k selector.
  [EB]   elebank, "DeepSeek-V4 explained", 模型創新 item 1 -- CSA and HCA interleaved,
         many tokens' KV become one KV entry.

The pages give no formula for the pooling, the indexer score or the attention.  The
readings taken here (each is marked READING in the function that uses it):
  R1  pooling: a softmax-weighted sum over each block of r tokens with per-position
      weights omega (shared by all blocks and channels); the tail of T mod r tokens is
      not pooled.
  R2  indexer score: s_j = sum_g w_g * max(0, q_g . c_j) (the published DSA lightning
      indexer form), computed exactly, rounded to fp32, then to bf16 when bf16 scores are
      requested (the pages: FP32 scores compressed to BF16).  -0 is taken as +0.
  R3  top-k: the min(k, n) visible entries with the largest score, ties to the lowest
      index; output ascending, padded with -1.
  R4  CSA attention: one softmax over the selected compressed entries followed by the
      raw window tokens [max(0, p-w+1), p]; no de-duplication of the overlap.
  R5  HCA attention: one softmax over every visible HCA entry; no window.
  R6  visibility: entry j (block of r tokens) is visible to the token at position p iff
      (j+1)*r <= p+1, i.e. n(p) = min(N, floor((p+1)/r)).
  R7  MXFP4 (OCP Microscaling v1.0, e2m1 elements, e8m0 scale per 32 elements): scale
      exponent floor(log2(amax)) - 2, element = round-to-nearest-even of v / 2^e onto the
      e2m1 grid, saturating at +-6; amax = 0 gives exponent -127 and zero elements.
  (R8-R10 -- heads and scale, positions, layer order -- concern the callers, not this module.)
  R11 training (the sparse attention is trained from the 64K stage of the length
      curriculum [LH 八.2]): the gradients are those of the forward functions above, the
      exact derivative of softmax attention and of the pooled sum; the selection (top-k)
      is held fixed (not differentiated) and a rounding to the storage type passes the
      gradient unchanged.
"""

import math

import numpy as np

CSA_RATIO = 4        # [LH] 八.3 m = 4; [TL] every 4 tokens -> one block
HCA_RATIO = 128      # [LH] 八.3 m' = 128; [TL] every 128 tokens -> one entry
N_WIN = 128          # [LH] 八.3 sliding-window branch n_win = 128
TOPK_PRO = 1024      # [LH] 八.3 top-k = 1024 (Pro)
TOPK_FLASH = 512     # [LH] 八.3 top-k = 512 (Flash)
MX_BLOCK = 32        # OCP MX v1.0: 32 elements share one e8m0 scale


# --------------------------------------------------------------------------- rounding

def _round_binary(x, sig_bits, emin, emax):
    """Round float64 values to the nearest value of a binary floating-point format with
    `sig_bits` significand bits (implicit bit included), minimum normal exponent `emin`
    and maximum exponent `emax`; ties to even, gradual underflow, overflow to +-inf."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2**e with 0.5 <= |m| < 1
    quantum_exp = np.maximum(e - sig_bits, emin + 1 - sig_bits)
    y = np.ldexp(np.round(np.ldexp(x, -quantum_exp)), quantum_exp)  # np.round: half to even
    max_finite = (2.0 - 2.0 ** (1 - sig_bits)) * 2.0 ** emax
    return np.where(np.abs(y) > max_finite, np.copysign(np.inf, x), y)


def round_fp32(x):
    """Nearest IEEE binary32 value (round to nearest, ties to even), kept in float64."""
    return _round_binary(x, 24, -126, 127)


def round_bf16(x):
    """Nearest bfloat16 value (8 significand bits, binary32 exponent range), kept in float64."""
    return _round_binary(x, 8, -126, 127)


def round_to(x, dtype):
    """Round once to the storage type named by `dtype` ("f32" or "bf16")."""
    if dtype == "f32":
        return round_fp32(x)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------- MXFP4

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # magnitudes of codes 0..7


def mxfp4_quantize(v):
    """OCP MX FP4 (E2M1) quantization of the last axis in blocks of 32 [9F item 4 names FP4
    on the indexer QK path; the block format is READING R7].

    v: float64 array [..., D] with D a multiple of 32.
    Returns (codes uint8 [..., D] with sign in bit 3 and magnitude code in bits 0..2,
             scale_exp int [..., D/32] in [-127, 127]).
    """
    v = np.asarray(v, dtype=np.float64)
    D = v.shape[-1]
    assert D % MX_BLOCK == 0
    blocks = v.reshape(v.shape[:-1] + (D // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(amax)                    # amax = m * 2**e, so floor(log2 amax) = e - 1
    scale_exp = np.where(amax > 0, np.clip((e - 1) - 2, -127, 127), -127)
    t = np.abs(blocks) / np.ldexp(1.0, scale_exp)[..., None]
    dist = np.abs(t[..., None] - E2M1_GRID)  # distance to every grid point
    nearest = dist == dist.min(axis=-1, keepdims=True)
    first = np.argmax(nearest, axis=-1)
    tie = nearest.sum(axis=-1) == 2          # a tie is between codes first and first + 1
    mag = np.where(tie & (first % 2 == 1), first + 1, first)
    sign = np.signbit(blocks).astype(np.int64)
    codes = (sign << 3) | mag
    return codes.reshape(v.shape).astype(np.uint8), scale_exp.astype(np.int64)


def mxfp4_dequantize(codes, scale_exp):
    """Exact float64 values of MXFP4 codes [..., D] with scale exponents [..., D/32]."""
    codes = np.asarray(codes).astype(np.int64)
    D = codes.shape[-1]
    mag = E2M1_GRID[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    scale = np.repeat(np.ldexp(1.0, np.asarray(scale_exp)), MX_BLOCK, axis=-1)
    return val * scale.reshape(codes.shape[:-1] + (D,))


def mxfp4_pack(codes):
    """Two codes per byte: element 2i in the low nibble, element 2i+1 in the high nibble."""
    codes = np.asarray(codes).astype(np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def mxfp4_unpack(packed):
    packed = np.asarray(packed).astype(np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------- compression

def pool_weights(omega):
    """Softmax of the per-position pooling logits omega [r] (READING R1)."""
    omega = np.asarray(omega, dtype=np.float64)
    a = np.exp(omega - omega.max())
    return a / a.sum()


def compress(x, omega, ratio):
    """Pool every `ratio` consecutive tokens into one entry [LH 八.3; TL; EB; READING R1].

    x: float64 [T, D] (the stored values, widened exactly).
    Returns float64 [floor(T/ratio), D], unrounded.
    """
    x = np.asarray(x, dtype=np.float64)
    alpha = pool_weights(omega)
    assert alpha.shape == (ratio,)
    n = x.shape[0] // ratio
    blocks = x[: n * ratio].reshape(n, ratio, x.shape[1])
    return np.einsum("jid,i->jd", blocks, alpha)


def entry_count(T, ratio):
    """Number of compressed entries a context of T tokens holds."""
    return T // ratio


def visible_entries(p, N, ratio):
    """Entries visible to the token at position p (READING R6)."""
    return min(N, (p + 1) // ratio)


def window_positions(p, n_win):
    """Positions of the sliding window ending at (and including) p [LH 八.3; READING R4]."""
    return np.arange(max(0, p - n_win + 1), p + 1)


# --------------------------------------------------------------------------- indexer + top-k

def index_scores(q_idx, w_idx, k_idx, n_visible, score_dtype):
    """Lightning-indexer scores of the first n_visible compressed keys [LH 八.3, 八.7;
    9F item 4; READING R2].

    q_idx [H_I, d_I], w_idx [H_I], k_idx [N, d_I]: float64 (exact stored values).
    Returns float64 [n_visible] holding fp32 (or bf16) representable values.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w_idx = np.asarray(w_idx, dtype=np.float64)
    keys = np.asarray(k_idx, dtype=np.float64)[:n_visible]
    dots = keys @ q_idx.T                    # [n, H_I]
    s = np.maximum(dots, 0.0) @ w_idx        # [n]
    s = round_fp32(s)
    if score_dtype == "bf16":
        s = round_bf16(s)
    elif score_dtype != "f32":
        raise ValueError(score_dtype)
    return s + 0.0                           # -0 -> +0


def select_topk(scores, n_visible, k):
    """Top-k selector [LH 八.3; READING R3]: the min(k, n) largest of scores[:n], ties to
    the lowest index, returned ascending and padded with -1 to length k."""
    s = np.asarray(scores, dtype=np.float64)[:n_visible]
    order = np.lexsort((np.arange(n_visible), -s))   # by score desc, then index asc
    chosen = np.sort(order[: min(k, n_visible)])
    out = np.full(k, -1, dtype=np.int64)
    out[: chosen.size] = chosen
    return out


# --------------------------------------------------------------------------- attention

def attend(q, keys, values, scale):
    """Softmax attention of every head of q [H, d] over keys/values [L, d].
    Returns (o [H, d], lse [H]); an empty key list gives o = 0, lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    H, d = q.shape
    if keys.shape[0] == 0:
        return np.zeros((H, d)), np.full(H, -np.inf)
    logits = scale * (q @ np.asarray(keys, dtype=np.float64).T)      # [H, L]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    denom = e.sum(axis=1, keepdims=True)
    o = (e @ np.asarray(values, dtype=np.float64)) / denom
    lse = (m + np.log(denom))[:, 0]
    return o, lse


def csa_keys(Kc, Vc, idx, K_raw, V_raw, raw_pos0, p, n_win, n_visible):
    """Key/value list of one CSA query: selected compressed entries (ascending), then the
    raw window tokens [LH 八.3; READINGS R4, R6].  Indices outside [0, n_visible) are
    padding and are skipped."""
    sel = [int(j) for j in idx if 0 <= j < n_visible]
    win = window_positions(p, n_win) - raw_pos0
    keys = np.concatenate([np.asarray(Kc, np.float64)[sel], np.asarray(K_raw, np.float64)[win]])
    vals = np.concatenate([np.asarray(Vc, np.float64)[sel], np.asarray(V_raw, np.float64)[win]])
    return keys, vals


def csa_attention(q, Kc, Vc, idx, K_raw, V_raw, raw_pos0, p, n_win, scale, ratio=CSA_RATIO):
    """CSA sparse attention of one query token at position p (READINGS R4, R6)."""
    n_vis = visible_entries(p, Kc.shape[0], ratio)
    keys, vals = csa_keys(Kc, Vc, idx, K_raw, V_raw, raw_pos0, p, n_win, n_vis)
    return attend(q, keys, vals, scale)


def hca_attention(q, Kh, Vh, p, scale, ratio=HCA_RATIO):
    """HCA dense attention of one query token at position p [LH 八.3; READINGS R5, R6]."""
    n = visible_entries(p, Kh.shape[0], ratio)
    return attend(q, Kh[:n], Vh[:n], scale)


def lse_merge(o_parts, lse_parts):
    """Combine partial attentions over disjoint key sets: o = sum_s e^(lse_s - L) o_s with
    L = log sum_s e^(lse_s).  o_parts [S, H, d], lse_parts [S, H]."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.exp(lse_parts - m_safe)                        # [S, H]
    tot = w.sum(axis=0)
    L = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    o = np.where(finite[:, None], (w[:, :, None] * o_parts).sum(axis=0)
                 / np.where(finite, tot, 1.0)[:, None], 0.0)
    return o, L


# --------------------------------------------------------------------------- one query, end to end

def decode_query(q, q_idx, w_idx, Kc, Vc, Ic, K_raw, V_raw, raw_pos0, Kh, Vh, p, topk,
                 n_win, scale, score_dtype):
    """One query token at position p through one CSA layer and one HCA layer.

    Ic holds the indexer keys exactly as stored (already MXFP4-dequantized when the
    indexer runs in MXFP4).  Returns a dict with scores, idx, csa (o, lse), hca (o, lse).
    """
    n_c = visible_entries(p, Kc.shape[0], CSA_RATIO)
    scores = index_scores(q_idx, w_idx, Ic, n_c, score_dtype)
    idx = select_topk(scores, n_c, topk)
    csa = csa_attention(q, Kc, Vc, idx, K_raw, V_raw, raw_pos0, p, n_win, scale)
    hca = hca_attention(q, Kh, Vh, p, scale)
    return {"scores": scores, "idx": idx, "csa": csa, "hca": hca}


def mxfp4_roundtrip(v):
    """Value an MXFP4 encode/decode of v produces (what the indexer sees in MXFP4 mode)."""
    codes, se = mxfp4_quantize(v)
    return mxfp4_dequantize(codes, se)


def softmax_weights(q, keys, scale):
    """Attention probabilities of each head (rows sum to one); used by the pins."""
    logits = scale * (np.asarray(q, np.float64) @ np.asarray(keys, np.float64).T)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def log2_floor(x):
    """floor(log2 x) for x > 0, exactly."""
    return math.frexp(x)[1] - 1


# --------------------------------------------------------------------------- backward (READING R11)

def attend_backward(q, keys, values, scale, dout, dlse=None):
    """Gradients of attend(q, keys, values, scale) for the loss sum(dout * o) +
    sum(dlse * lse): returns (dq [H, d], dkeys [L, d], dvalues [L, d]).  With the
    probabilities P = softmax(scale q k^T) of each head: dvalues = P^T dout,
    dS = P (dout v^T - rowsum(dout * o) + dlse), dq = scale dS keys, dkeys = scale dS^T q.
    An empty key list gives dq = 0."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    H, d = q.shape
    if keys.shape[0] == 0:
        return np.zeros((H, d)), np.zeros((0, d)), np.zeros((0, d))
    P = softmax_weights(q, keys, scale)                  # [H, L]
    o = P @ values                                       # [H, d]
    dP = dout @ values.T                                 # [H, L]
    rowterm = (dout * o).sum(axis=1, keepdims=True)      # [H, 1]
    if dlse is not None:
        rowterm = rowterm - np.asarray(dlse, dtype=np.float64)[:, None]
    dS = P * (dP - rowterm)
    return scale * dS @ keys, scale * dS.T @ q, P.T @ dout


def csa_attention_backward(q, Kc, Vc, idx, K_raw, V_raw, raw_pos0, p, n_win, scale, dout,
                           dlse=None, ratio=CSA_RATIO):
    """Gradients of csa_attention for one query token (READINGS R4, R6, R11): dq [H, d], and
    the contributions to the compressed entries dKc, dVc (shape of Kc) and to the raw rows
    dK_raw, dV_raw (shape of K_raw), each key's gradient added to the row it came from."""
    n_vis = visible_entries(p, Kc.shape[0], ratio)
    keys, vals = csa_keys(Kc, Vc, idx, K_raw, V_raw, raw_pos0, p, n_win, n_vis)
    dq, dk, dv = attend_backward(q, keys, vals, scale, dout, dlse)
    sel = [int(j) for j in idx if 0 <= j < n_vis]
    win = window_positions(p, n_win) - raw_pos0
    dKc = np.zeros(np.shape(Kc))
    dVc = np.zeros(np.shape(Vc))
    dKr = np.zeros(np.shape(K_raw))
    dVr = np.zeros(np.shape(V_raw))
    ns = len(sel)
    np.add.at(dKc, sel, dk[:ns])
    np.add.at(dVc, sel, dv[:ns])
    np.add.at(dKr, win, dk[ns:])
    np.add.at(dVr, win, dv[ns:])
    return dq, dKc, dVc, dKr, dVr


def hca_attention_backward(q, Kh, Vh, p, scale, dout, dlse=None, ratio=HCA_RATIO):
    """Gradients of hca_attention for one query token (READINGS R5, R6, R11): dq, dKh, dVh
    (the entries past the visible count get zero)."""
    n = visible_entries(p, Kh.shape[0], ratio)
    dq, dk, dv = attend_backward(q, Kh[:n], Vh[:n], scale, dout, dlse)
    dKh = np.zeros(np.shape(Kh))
    dVh = np.zeros(np.shape(Vh))
    dKh[:n] = dk
    dVh[:n] = dv
    return dq, dKh, dVh


def compress_backward(x, omega, ratio, dy):
    """Gradients of sum(dy * compress(x, omega, ratio)) (READINGS R1, R11): dx [T, D] (token
    j*ratio + i gets alpha_i dy[j]; the unpooled tail gets zero) and domega [ratio]
    (domega_k = alpha_k (g_k - sum_i alpha_i g_i) with g_i = sum_j dy[j] . x[j*ratio + i],
    the softmax's derivative)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    alpha = pool_weights(omega)
    n = x.shape[0] // ratio
    dx = np.zeros_like(x)
    dx[: n * ratio] = (alpha[None, :, None] * dy[:n, None, :]).reshape(n * ratio, x.shape[1])
    blocks = x[: n * ratio].reshape(n, ratio, x.shape[1])
    g = np.einsum("jid,jd->i", blocks, dy[:n])
    domega = alpha * (g - (alpha * g).sum())
    return dx, domega
