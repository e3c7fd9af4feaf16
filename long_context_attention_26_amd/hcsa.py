"""ctypes binding of libhcsa (the C ABI in include/hcsa.h).

Argument marshalling only: every step runs in the library's HIP kernels.  Tensors must be
on the GPU; their data pointers and the current torch stream are handed to the library.
Importing this module fails loudly when the library has not been built.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhcsa.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with "
                      "`python long_context_attention_26_amd/build.py`")
lib = ctypes.CDLL(_LIB_PATH)

F32, BF16, MXFP4, MXFP4_FP8 = 0, 1, 2, 3
OK, EINVAL, EDTYPE, EALIGN, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5

_p, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "hcsa_version": (_i, []),
    "hcsa_last_error": (ctypes.c_char_p, []),
    "hcsa_time_next_indexer": (_i, [_p, _p]),
    "hcsa_set_attn_splits": (_i, [_i]),
    "hcsa_compress_kv": (_i, [_p, _i, _i64, _i, _i, _i, _p, _i, _p, _i, _i64, _p, _i64, _p]),
    "hcsa_compress_kv_batched": (_i, [_p, _i, _i, _p, _p]),
    "hcsa_mxfp4_quantize": (_i, [_p, _i, _i64, _i, _p, _p, _p]),
    "hcsa_topk_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "hcsa_topk": (_i, [_p, _i, _i64, _i, _i, _i, _i, _i64, _p, _i, _p, _p, _sz, _p]),
    "hcsa_csa_hca_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "hcsa_csa_hca_attn": (_i, [_p, _p, _p, _i64, _i, _p, _i, _p, _p, _i64, _i64, _i64, _i, _i,
                               _p, _p, _i64, _i, _i, _i64, _p, _p, _i, _i, _i, _i, _i, _f, _p,
                               _p, _p, _p, _p, _sz, _p]),
    "hcsa_csa_sparse_attn_bwd_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "hcsa_csa_sparse_attn_bwd": (_i, [_p, _p, _p, _i64, _i, _p, _i, _p, _p, _i64, _i64, _i64,
                                      _i, _i, _i64, _p, _i, _i, _i, _i, _i, _f, _p, _p, _p,
                                      _p, _p, _p, _p, _i64, _p, _p, _i64, _p, _sz, _p]),
    "hcsa_hca_dense_attn_bwd_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "hcsa_hca_dense_attn_bwd": (_i, [_p, _p, _p, _i64, _i, _i, _i64, _p, _i, _i, _i, _i, _i,
                                     _f, _p, _p, _p, _p, _p, _p, _p, _i64, _p, _sz, _p]),
    "hcsa_compress_kv_bwd_workspace_size": (_sz, [_i, _i, _i]),
    "hcsa_compress_kv_bwd": (_i, [_p, _i, _i64, _i, _i, _i, _p, _i, _p, _i64, _p, _i64, _p, _p,
                                  _sz, _p]),
    "hcsa_csa_index_topk_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "hcsa_csa_index_topk": (_i, [_p, _i, _p, _p, _i, _i64, _p, _i64, _i, _i, _i, _i, _i, _i,
                                 _i64, _p, _p, _i, _i, _p, _p, _p, _sz, _p]),
    "hcsa_csa_pool_index_topk": (_i, [_p, _i, _p, _i, _p, _p, _i, _i64, _p, _i64, _i, _i,
                                      _i, _i, _i, _i, _i64, _p, _p, _i, _i, _p, _p, _p, _sz,
                                      _p]),
    "hcsa_csa_index_scores": (_i, [_p, _i, _p, _p, _i, _i64, _p, _i64, _i, _i, _i, _i, _i, _i,
                                   _i64, _p, _p, _i, _p, _p]),
    "hcsa_csa_sparse_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "hcsa_csa_sparse_attn": (_i, [_p, _p, _p, _i64, _i, _p, _i, _p, _p, _i64, _i64, _i64, _i,
                                  _i, _i64, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p, _p, _sz,
                                  _p]),
    "hcsa_hca_dense_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "hcsa_decode_step_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "hcsa_decode_step": (_i, [_p, _i, _p, _i, _p, _p, _i, _i64, _p, _i64, _i, _i, _i, _p,
                              _p, _p, _p, _i64, _i, _i, _p, _p, _i64, _i64, _i64, _i, _i,
                              _p, _p, _i64, _i, _i, _i64, _p, _p, _i, _i, _i, _i, _i, _f,
                              _p, _p, _p, _p, _p, _sz, _p]),
    "hcsa_decode_step_noalloc": (_i, [_p, _i, _p, _i, _p, _p, _i, _i64, _p, _i64, _i, _i, _i,
                                      _p, _p, _p, _p, _i64, _i, _i, _p, _p, _i64, _i64, _i64,
                                      _i, _i, _p, _p, _i64, _i, _i, _i64, _p, _p, _i, _i, _i,
                                      _i, _i, _f, _p, _p, _p, _p, _p]),
    "hcsa_hca_dense_attn": (_i, [_p, _p, _p, _i64, _i, _i, _i64, _p, _p, _i, _i, _i, _i, _i,
                                 _f, _p, _p, _p, _sz, _p]),
}
MAX_POOL_JOBS = 8
DECODE_STEP_SCRATCH_BYTES = 128 << 20    # HCSA_DECODE_STEP_SCRATCH_BYTES


class PoolJob(ctypes.Structure):
    """Mirror of struct hcsa_pool_job."""
    _fields_ = [("x", _p), ("x_dtype", _i), ("x_bstride", _i64), ("T", _i), ("D", _i),
                ("omega", _p), ("ratio", _i), ("y", _p), ("y_dtype", _i), ("y_bstride", _i64),
                ("y_scales", _p), ("ys_bstride", _i64), ("pos0", _i64)]


class Pages(ctypes.Structure):
    """Mirror of struct hcsa_pages."""
    _fields_ = [("block_table", _p), ("table_stride", _i64), ("raw_ring", _i64)]


def _pages(table, raw_ring=0):
    """hcsa_pages for a block table (int32 [B, max_blocks] device tensor) and/or a raw-token
    ring of raw_ring rows, or None for contiguous caches."""
    if table is None and not raw_ring:
        return None
    if table is not None and (table.dtype != torch.int32 or table.dim() != 2
                              or table.stride(1) != 1):
        raise ValueError("the block table must be an int32 [B, max_blocks] tensor with unit "
                         "column stride")
    if table is None:
        return ctypes.byref(Pages(None, 0, raw_ring))
    return ctypes.byref(Pages(table.data_ptr(), table.stride(0), raw_ring))


for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class HcsaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"hcsa error {code}: {msg}")
        self.code = code


def _check(rc):
    if rc != OK:
        raise HcsaError(rc, lib.hcsa_last_error().decode())
    return rc


def dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _pos_ptr(seq_pos, B):
    """Device pointer of an int64 [B] per-sequence position tensor, or None."""
    if seq_pos is None:
        return None
    if seq_pos.dtype != torch.int64 or seq_pos.numel() != B or not seq_pos.is_contiguous():
        raise ValueError("seq_pos must be a contiguous int64 tensor of B positions")
    return seq_pos.data_ptr()


def time_next_indexer(start_event, stop_event):
    """The next indexer kernel launched by this thread records these torch.cuda.Events
    (timing enabled) as part of its dispatch."""
    for e in (start_event, stop_event):
        if e.cuda_event == 0:
            e.record()          # creates the underlying event
    _check(lib.hcsa_time_next_indexer(start_event.cuda_event, stop_event.cuda_event))


def set_attn_splits(splits):
    """Split count of this thread's later attention calls (0: each call chooses)."""
    _check(lib.hcsa_set_attn_splits(int(splits)))


def alloc_workspace(nbytes, device):
    """Caller-owned workspace (torch's allocator returns 512-byte aligned blocks)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def compress_kv(x, omega, ratio, y, y_scales=None, stream=None):
    """Pool every `ratio` rows of x [B, T, D] into y [B, >= T//ratio, D] (F32/BF16), or into
    packed MXFP4 codes y uint8 [B, n, D/2] with scales y_scales uint8 [B, n, D/32]."""
    B, T, D = x.shape
    assert x.stride(2) == 1 and x.stride(1) == D
    if y.dtype == torch.uint8:
        y_dt = MXFP4
        assert y_scales is not None and y.stride(2) == 1 and y_scales.stride(2) == 1
        ysb = y_scales.stride(0)
    else:
        y_dt = dtype_code(y)
        ysb = 0
    _check(lib.hcsa_compress_kv(_ptr(x), dtype_code(x), x.stride(0), B, T, D, _ptr(omega),
                                ratio, _ptr(y), y_dt, y.stride(0), _ptr(y_scales), ysb,
                                _stream(stream)))
    return y


def pool_job(x, omega, ratio, y, y_scales=None, T=None, pos0=0):
    """Describe one pooling job (same tensor conventions as compress_kv).  For paged caches
    x and y are page pools ([pages, 128, D] and [pages, 128/ratio, ...]) and the job pools
    tokens [pos0, pos0 + T) of every sequence."""
    D = x.shape[-1]
    assert x.stride(-1) == 1 and x.stride(-2) == D
    if T is None:
        T = x.shape[1]
    if y.dtype == torch.uint8:
        y_dt, ysb = MXFP4, y_scales.stride(0)
    else:
        y_dt, ysb = dtype_code(y), 0
    return PoolJob(_ptr(x), dtype_code(x), x.stride(0), T, D, _ptr(omega), ratio, _ptr(y), y_dt,
                   y.stride(0), _ptr(y_scales), ysb, pos0)


def compress_kv_batched(jobs, B, stream=None, block_table=None, raw_ring=0):
    """Run up to MAX_POOL_JOBS pooling jobs (from pool_job) of one batch in one launch;
    block_table (int32 [B, max_blocks]) selects paged caches, raw_ring > 0 raw tokens (the
    jobs' x) in a ring of that many rows per sequence."""
    arr = (PoolJob * max(1, len(jobs)))(*jobs)
    _check(lib.hcsa_compress_kv_batched(ctypes.cast(arr, _p), len(jobs), B,
                                        _pages(block_table, raw_ring), _stream(stream)))


def mxfp4_quantize(x, packed, scales, stream=None):
    """Quantize rows of x [..., D] into packed [..., D/2] and scales [..., D/32] (uint8)."""
    D = x.shape[-1]
    rows = x.numel() // D
    _check(lib.hcsa_mxfp4_quantize(_ptr(x), dtype_code(x), rows, D, _ptr(packed),
                                   _ptr(scales), _stream(stream)))
    return packed, scales


def topk_workspace_size(score_dtype, B, Nq, N, k):
    return lib.hcsa_topk_workspace_size(score_dtype, B, Nq, N, k)


def topk(scores, B, Nq, N, ratio, pos0, k, idx, workspace=None, stream=None, seq_pos=None):
    """Select per row of scores [B*Nq, row_stride] (F32/BF16) into idx int32 [B*Nq, k].
    seq_pos: optional int64 [B] device tensor of per-sequence positions (ragged batches)."""
    sdt = dtype_code(scores)
    if workspace is None:
        workspace = alloc_workspace(topk_workspace_size(sdt, B, Nq, N, k), scores.device)
    _check(lib.hcsa_topk(_ptr(scores), sdt, scores.stride(0), B, Nq, N, ratio, pos0,
                         _pos_ptr(seq_pos, B), k, _ptr(idx), _ptr(workspace), workspace.numel(),
                         _stream(stream)))
    return idx


def index_topk_workspace_size(B, Nq, N, k, score_dtype):
    return lib.hcsa_csa_index_topk_workspace_size(B, Nq, N, k, score_dtype)


def csa_index_topk(q_idx, w_idx, k_idx, N, ratio, pos0, k, score_dtype, topk_idx,
                   k_scales=None, scores_out=None, workspace=None, stream=None, seq_pos=None,
                   block_table=None, mx_fp8=False):
    """q_idx [B, Nq, H_I, d_I], w_idx [B, Nq, H_I] f32, k_idx [B, >=N, d_I] (F32/BF16) or
    packed MXFP4 uint8 [B, >=N, d_I/2] with k_scales [B, >=N, d_I/32].  mx_fp8: scan MXFP4
    keys on FP8 operands (the codes widened to e4m3) instead of FP4 ones."""
    B, Nq, H_I, d_I = q_idx.shape
    if k_idx.dtype == torch.uint8:
        k_dt, ksb = (MXFP4_FP8 if mx_fp8 else MXFP4), k_scales.stride(0)
    else:
        k_dt, ksb = dtype_code(k_idx), 0
    if workspace is None:
        workspace = alloc_workspace(index_topk_workspace_size(B, Nq, N, k, score_dtype),
                                    q_idx.device)
    _check(lib.hcsa_csa_index_topk(_ptr(q_idx), dtype_code(q_idx), _ptr(w_idx), _ptr(k_idx),
                                   k_dt, k_idx.stride(0), _ptr(k_scales), ksb, B, Nq, H_I,
                                   d_I, N, ratio, pos0, _pos_ptr(seq_pos, B),
                                   _pages(block_table), k, score_dtype, _ptr(topk_idx),
                                   _ptr(scores_out), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))
    return topk_idx


def csa_pool_index_topk(jobs, q_idx, w_idx, k_idx, N, ratio, pos0, k, score_dtype, topk_idx,
                        k_scales=None, scores_out=None, workspace=None, stream=None,
                        seq_pos=None, block_table=None, raw_ring=0, mx_fp8=False):
    """compress_kv_batched(jobs, ...) then csa_index_topk(...) as one call (the pooling runs
    in the launch of the selection's per-row floors when the scores are not stored)."""
    B, Nq, H_I, d_I = q_idx.shape
    if k_idx.dtype == torch.uint8:
        k_dt, ksb = (MXFP4_FP8 if mx_fp8 else MXFP4), k_scales.stride(0)
    else:
        k_dt, ksb = dtype_code(k_idx), 0
    if workspace is None:
        workspace = alloc_workspace(index_topk_workspace_size(B, Nq, N, k, score_dtype),
                                    q_idx.device)
    arr = (PoolJob * max(1, len(jobs)))(*jobs)
    _check(lib.hcsa_csa_pool_index_topk(ctypes.cast(arr, _p), len(jobs), _ptr(q_idx),
                                        dtype_code(q_idx), _ptr(w_idx), _ptr(k_idx), k_dt,
                                        k_idx.stride(0), _ptr(k_scales), ksb, B, Nq, H_I, d_I,
                                        N, ratio, pos0, _pos_ptr(seq_pos, B),
                                        _pages(block_table, raw_ring), k, score_dtype,
                                        _ptr(topk_idx), _ptr(scores_out), _ptr(workspace),
                                        workspace.numel(), _stream(stream)))
    return topk_idx


def decode_step_workspace_size(B, Nq, N, k, score_dtype, H, d, n_win, N_h):
    return lib.hcsa_decode_step_workspace_size(B, Nq, N, k, score_dtype, H, d, n_win, N_h)


def _decode_step_args(jobs, q_idx, w_idx, k_idx, score_dtype, topk_idx, q, kc, vc, N, k,
                      k_raw, v_raw, raw_pos0, n_win, ratio, kh, vh, N_h, ratio_h, pos0, scale,
                      out_c, lse_c, out_h, lse_h, k_scales, seq_pos, block_table, raw_ring,
                      mx_fp8):
    """The step's arguments up to lse_h, as the C calls take them (the first is the pool-job
    array, which must stay referenced until the call returns)."""
    B, Nq, H_I, d_I = q_idx.shape
    _, _, H, d = q.shape
    if k_idx.dtype == torch.uint8:
        k_dt, ksb = (MXFP4_FP8 if mx_fp8 else MXFP4), k_scales.stride(0)
    else:
        k_dt, ksb = dtype_code(k_idx), 0
    arr = (PoolJob * max(1, len(jobs)))(*jobs)
    return (arr, len(jobs), _ptr(q_idx), dtype_code(q_idx), _ptr(w_idx),
            _ptr(k_idx), k_dt, k_idx.stride(0), _ptr(k_scales), ksb, H_I, d_I, score_dtype,
            _ptr(topk_idx), _ptr(q), _ptr(kc), _ptr(vc), kc.stride(0), N, k, _ptr(k_raw),
            _ptr(v_raw), k_raw.stride(0) if k_raw is not None else 0,
            k_raw.shape[1] if k_raw is not None else 0, raw_pos0, n_win, ratio, _ptr(kh),
            _ptr(vh), kh.stride(0), N_h, ratio_h, pos0, _pos_ptr(seq_pos, B),
            _pages(block_table, raw_ring), dtype_code(q), B, Nq, H, d, scale, _ptr(out_c),
            _ptr(lse_c), _ptr(out_h), _ptr(lse_h))


def decode_step(jobs, q_idx, w_idx, k_idx, score_dtype, topk_idx, q, kc, vc, N, k, k_raw,
                v_raw, raw_pos0, n_win, ratio, kh, vh, N_h, ratio_h, pos0, scale, out_c,
                lse_c, out_h, lse_h, k_scales=None, workspace=None, stream=None,
                seq_pos=None, block_table=None, raw_ring=0, mx_fp8=False):
    """One decode step: csa_pool_index_topk(jobs, ...) then csa_hca_attn(...) as one call
    (same results).  q_idx [B, Nq, H_I, d_I]; q [B, Nq, H, d]; the indexer shares N and
    ratio with CSA."""
    B, Nq = q_idx.shape[:2]
    H, d = q.shape[2:]
    if workspace is None:
        workspace = alloc_workspace(decode_step_workspace_size(B, Nq, N, k, score_dtype, H, d,
                                                               n_win, N_h), q.device)
    args = _decode_step_args(jobs, q_idx, w_idx, k_idx, score_dtype, topk_idx, q, kc, vc, N,
                             k, k_raw, v_raw, raw_pos0, n_win, ratio, kh, vh, N_h, ratio_h,
                             pos0, scale, out_c, lse_c, out_h, lse_h, k_scales, seq_pos,
                             block_table, raw_ring, mx_fp8)
    _check(lib.hcsa_decode_step(ctypes.cast(args[0], _p), *args[1:], _ptr(workspace),
                                workspace.numel(), _stream(stream)))
    return topk_idx


def decode_step_noalloc(jobs, q_idx, w_idx, k_idx, score_dtype, topk_idx, q, kc, vc, N, k,
                        k_raw, v_raw, raw_pos0, n_win, ratio, kh, vh, N_h, ratio_h, pos0,
                        scale, out_c, lse_c, out_h, lse_h, k_scales=None, stream=None,
                        seq_pos=None, block_table=None, raw_ring=0, mx_fp8=False):
    """decode_step with the library's fixed per-GPU scratch as its workspace: nothing is
    allocated (steps needing up to DECODE_STEP_SCRATCH_BYTES of workspace; calls that
    overlap on one GPU race)."""
    args = _decode_step_args(jobs, q_idx, w_idx, k_idx, score_dtype, topk_idx, q, kc, vc, N,
                             k, k_raw, v_raw, raw_pos0, n_win, ratio, kh, vh, N_h, ratio_h,
                             pos0, scale, out_c, lse_c, out_h, lse_h, k_scales, seq_pos,
                             block_table, raw_ring, mx_fp8)
    _check(lib.hcsa_decode_step_noalloc(ctypes.cast(args[0], _p), *args[1:], _stream(stream)))
    return topk_idx


def csa_index_scores(q_idx, w_idx, k_idx, N, ratio, pos0, scores, k_scales=None, stream=None,
                     seq_pos=None, block_table=None, mx_fp8=False):
    """Indexer scores only, into scores [B*Nq, N] (F32 or BF16)."""
    B, Nq, H_I, d_I = q_idx.shape
    if k_idx.dtype == torch.uint8:
        k_dt, ksb = (MXFP4_FP8 if mx_fp8 else MXFP4), k_scales.stride(0)
    else:
        k_dt, ksb = dtype_code(k_idx), 0
    _check(lib.hcsa_csa_index_scores(_ptr(q_idx), dtype_code(q_idx), _ptr(w_idx), _ptr(k_idx),
                                     k_dt, k_idx.stride(0), _ptr(k_scales), ksb, B, Nq, H_I,
                                     d_I, N, ratio, pos0, _pos_ptr(seq_pos, B),
                                     _pages(block_table), dtype_code(scores), _ptr(scores),
                                     _stream(stream)))
    return scores


def csa_attn_workspace_size(B, Nq, H, d, k, n_win):
    return lib.hcsa_csa_sparse_attn_workspace_size(B, Nq, H, d, k, n_win)


def csa_sparse_attn(q, kc, vc, N, topk_idx, k_raw, v_raw, raw_pos0, n_win, ratio, pos0, scale,
                    out, lse, workspace=None, stream=None, seq_pos=None, block_table=None,
                    raw_ring=0):
    """q [B, Nq, H, d]; kc, vc [B, >=N, d]; topk_idx [B, Nq, k]; k_raw, v_raw [B, T_raw, d]
    (with raw_ring > 0: rings [B, raw_ring, d], position t in row t % raw_ring)."""
    B, Nq, H, d = q.shape
    k = topk_idx.shape[-1]
    if workspace is None:
        workspace = alloc_workspace(csa_attn_workspace_size(B, Nq, H, d, k, n_win), q.device)
    _check(lib.hcsa_csa_sparse_attn(_ptr(q), _ptr(kc), _ptr(vc), kc.stride(0), N,
                                    _ptr(topk_idx), k, _ptr(k_raw), _ptr(v_raw),
                                    k_raw.stride(0), k_raw.shape[1], raw_pos0, n_win, ratio,
                                    pos0, _pos_ptr(seq_pos, B), _pages(block_table, raw_ring),
                                    dtype_code(q), B, Nq, H, d, scale, _ptr(out),
                                    _ptr(lse), _ptr(workspace), workspace.numel(),
                                    _stream(stream)))
    return out, lse


def csa_hca_attn_workspace_size(B, Nq, H, d, k, n_win, N_h):
    return lib.hcsa_csa_hca_attn_workspace_size(B, Nq, H, d, k, n_win, N_h)


def csa_hca_attn(q, kc, vc, N, topk_idx, k_raw, v_raw, raw_pos0, n_win, ratio, kh, vh, N_h,
                 ratio_h, pos0, scale, out_c, lse_c, out_h, lse_h, workspace=None, stream=None,
                 seq_pos=None, block_table=None, raw_ring=0):
    """csa_sparse_attn and hca_dense_attn of the same query tokens in one call (one launch
    on the decode fast path)."""
    B, Nq, H, d = q.shape
    k = topk_idx.shape[-1]
    if workspace is None:
        workspace = alloc_workspace(csa_hca_attn_workspace_size(B, Nq, H, d, k, n_win, N_h),
                                    q.device)
    _check(lib.hcsa_csa_hca_attn(_ptr(q), _ptr(kc), _ptr(vc), kc.stride(0), N, _ptr(topk_idx), k,
                                 _ptr(k_raw), _ptr(v_raw), k_raw.stride(0), k_raw.shape[1],
                                 raw_pos0, n_win, ratio, _ptr(kh), _ptr(vh), kh.stride(0), N_h,
                                 ratio_h, pos0, _pos_ptr(seq_pos, B),
                                 _pages(block_table, raw_ring), dtype_code(q), B, Nq, H, d,
                                 scale, _ptr(out_c), _ptr(lse_c), _ptr(out_h), _ptr(lse_h),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))
    return (out_c, lse_c), (out_h, lse_h)


def hca_attn_workspace_size(B, Nq, H, d, N):
    return lib.hcsa_hca_dense_attn_workspace_size(B, Nq, H, d, N)


def hca_dense_attn(q, kh, vh, N, ratio, pos0, scale, out, lse, workspace=None, stream=None,
                   seq_pos=None, block_table=None):
    """q [B, Nq, H, d]; kh, vh [B, >=N, d]."""
    B, Nq, H, d = q.shape
    if workspace is None:
        workspace = alloc_workspace(hca_attn_workspace_size(B, Nq, H, d, N), q.device)
    _check(lib.hcsa_hca_dense_attn(_ptr(q), _ptr(kh), _ptr(vh), kh.stride(0), N, ratio, pos0,
                                   _pos_ptr(seq_pos, B), _pages(block_table), dtype_code(q), B,
                                   Nq, H, d, scale, _ptr(out), _ptr(lse),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


# ------------------------------------------------------------------ backward (training)

def csa_sparse_attn_bwd(q, kc, vc, N, topk_idx, k_raw, v_raw, raw_pos0, n_win, ratio, pos0,
                        scale, out, lse, dout, dq, dkc, dvc, dk_raw, dv_raw, dlse=None,
                        workspace=None, stream=None, seq_pos=None,
                        key_major=True):
    """Backward of csa_sparse_attn: writes dq [B, Nq, H, d] f32; adds into dkc, dvc
    [B, >=N, d] f32 and dk_raw, dv_raw [B, T_raw, d] f32.
    key_major=False (with no workspace given) passes a null workspace: keys shared by
    consecutive tokens then get their gradients query-major, with atomics."""
    B, Nq, H, d = q.shape
    k = topk_idx.shape[-1]
    nbytes = lib.hcsa_csa_sparse_attn_bwd_workspace_size(B, Nq, H, d, dtype_code(q), N, k)
    if workspace is None and nbytes and key_major:
        workspace = alloc_workspace(nbytes, q.device)
    _check(lib.hcsa_csa_sparse_attn_bwd(_ptr(q), _ptr(kc), _ptr(vc), kc.stride(0), N,
                                        _ptr(topk_idx), k, _ptr(k_raw), _ptr(v_raw),
                                        k_raw.stride(0), k_raw.shape[1], raw_pos0, n_win, ratio,
                                        pos0, _pos_ptr(seq_pos, B), dtype_code(q), B, Nq, H, d,
                                        scale, _ptr(out), _ptr(lse), _ptr(dout), _ptr(dlse),
                                        _ptr(dq), _ptr(dkc), _ptr(dvc), dkc.stride(0),
                                        _ptr(dk_raw), _ptr(dv_raw), dk_raw.stride(0),
                                        _ptr(workspace),
                                        0 if workspace is None else workspace.numel(),
                                        _stream(stream)))
    return dq


def hca_dense_attn_bwd(q, kh, vh, N, ratio, pos0, scale, out, lse, dout, dq, dkh, dvh,
                       dlse=None, workspace=None, stream=None, seq_pos=None,
                       key_major=True):
    """Backward of hca_dense_attn: writes dq; adds into dkh, dvh [B, >=N, d] f32.
    key_major=False (with no workspace given) passes a null workspace: keys shared by
    consecutive tokens then get their gradients query-major, with atomics."""
    B, Nq, H, d = q.shape
    nbytes = lib.hcsa_hca_dense_attn_bwd_workspace_size(B, Nq, H, d, dtype_code(q))
    if workspace is None and nbytes and key_major:
        workspace = alloc_workspace(nbytes, q.device)
    _check(lib.hcsa_hca_dense_attn_bwd(_ptr(q), _ptr(kh), _ptr(vh), kh.stride(0), N, ratio, pos0,
                                       _pos_ptr(seq_pos, B), dtype_code(q), B, Nq, H, d, scale,
                                       _ptr(out), _ptr(lse), _ptr(dout), _ptr(dlse), _ptr(dq),
                                       _ptr(dkh), _ptr(dvh), dkh.stride(0), _ptr(workspace),
                                       0 if workspace is None else workspace.numel(),
                                       _stream(stream)))
    return dq


def compress_kv_bwd(x, omega, ratio, dy, dx, domega=None, workspace=None, stream=None):
    """Backward of compress_kv over x [B, T, D] (F32/BF16): adds into dx [B, T, D] f32 and,
    if given, domega [ratio] f32, from dy [B, T/ratio, D] f32."""
    B, T, D = x.shape
    if workspace is None:
        workspace = alloc_workspace(lib.hcsa_compress_kv_bwd_workspace_size(B, T, ratio),
                                    x.device)
    _check(lib.hcsa_compress_kv_bwd(_ptr(x), dtype_code(x), x.stride(0), B, T, D, _ptr(omega),
                                    ratio, _ptr(dy), dy.stride(0), _ptr(dx), dx.stride(0),
                                    _ptr(domega), _ptr(workspace), workspace.numel(),
                                    _stream(stream)))
    return dx, domega
