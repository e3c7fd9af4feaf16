"""One decode step / prefill chunk of a CSA layer and an HCA layer, as a sequence of
libhcsa calls on one stream (argument marshalling only; every step runs in HIP kernels).

Layout in HBM (all caller-owned torch tensors, row-major):
  raw K, V        [B, T, d]     kv dtype (the uncompressed tokens; the window reads the tail)
  raw indexer K   [B, T, d_I]   bf16 / f32
  CSA K, V        [B, T/4, d]   kv dtype           (pool ratio 4)
  indexer keys    [B, T/4, d_I] bf16 / f32, or MXFP4 codes [B, T/4, d_I/2] + scales
                  [B, T/4, d_I/32]
  HCA K, V        [B, T/128, d] kv dtype           (pool ratio 128)
Workspaces are allocated once per shape and reused by every step.
"""
import torch

from . import hcsa

R_CSA, R_HCA = 4, 128


class HybridAttentionState:
    """Caches of one CSA layer and one HCA layer for B sequences of capacity T tokens."""

    def clone_caches(self):
        """A state with private copies of the pooled caches that shares the raw tokens."""
        c = object.__new__(HybridAttentionState)
        c.__dict__.update(self.__dict__)
        for name in ("Kc", "Vc", "Kh", "Vh", "Ic", "Ics"):
            t = getattr(self, name)
            setattr(c, name, None if t is None else t.clone())
        return c

    def __init__(self, B, T, d, d_I, kv_dtype, idx_store, device, omegas):
        self.B, self.T, self.d, self.d_I = B, T, d, d_I
        self.kv_dtype = kv_dtype                      # torch.bfloat16 / torch.float32
        self.idx_store = idx_store                    # "f32" | "bf16" | "mxfp4"
        self.device = device
        self.omegas = omegas                          # dict of fp32 tensors on device
        Nc, Nh = T // R_CSA, T // R_HCA
        self.Nc, self.Nh = Nc, Nh
        e = lambda *s, dt=kv_dtype: torch.empty(*s, dtype=dt, device=device)
        self.Kc, self.Vc = e(B, Nc, d), e(B, Nc, d)
        self.Kh, self.Vh = e(B, Nh, d), e(B, Nh, d)
        if idx_store == "mxfp4":
            self.Ic = e(B, Nc, d_I // 2, dt=torch.uint8)
            self.Ics = e(B, Nc, d_I // 32, dt=torch.uint8)
        else:
            self.Ic = e(B, Nc, d_I, dt=torch.float32 if idx_store == "f32" else torch.bfloat16)
            self.Ics = None
        self.K_raw = self.V_raw = self.I_raw = None

    def attach_raw(self, K_raw, V_raw, I_raw):
        self.K_raw, self.V_raw, self.I_raw = K_raw, V_raw, I_raw

    def compress_range(self, t0, t1, stream=None):
        """Pool the CSA and HCA blocks whose last token lies in [t0, t1), all streams in
        one launch; each block is written at its own entry index."""
        jobs = self.pool_jobs(t0, t1)
        if jobs:
            hcsa.compress_kv_batched(jobs, self.B, stream=stream)

    def pool_jobs(self, t0, t1):
        """The pooling jobs of the CSA and HCA blocks whose last token lies in [t0, t1)."""
        jobs = []
        for ratio, pairs in ((R_CSA, ((self.K_raw, "csa_k", self.Kc), (self.V_raw, "csa_v", self.Vc),
                                      (self.I_raw, "idx_k", self.Ic))),
                             (R_HCA, ((self.K_raw, "hca_k", self.Kh), (self.V_raw, "hca_v", self.Vh)))):
            # block j covers tokens [j*ratio, (j+1)*ratio) and completes at its last token
            j0 = -(-(t0 + 1) // ratio) - 1
            j1 = t1 // ratio
            if j1 <= j0:
                continue
            for x, name, y in pairs:
                ys = self.Ics[:, j0:j1] if (y is self.Ic and self.Ics is not None) else None
                jobs.append(hcsa.pool_job(x[:, j0 * ratio: j1 * ratio], self.omegas[name], ratio,
                                          y[:, j0:j1], ys))
        return jobs


class DecodeStep:
    """Query token(s) at positions pos0 .. pos0+Nq-1 of every sequence through one CSA and
    one HCA layer.  Owns its outputs and workspaces."""

    def __init__(self, state, Nq, H, H_I, topk, n_win, score_dtype, scale):
        st = state
        self.st, self.Nq, self.H, self.H_I = st, Nq, H, H_I
        self.topk, self.n_win, self.scale = topk, n_win, scale
        self.mx_fp8 = False          # MXFP4 indexer keys: scan on FP8 operands instead of FP4
        self.score_code = hcsa.BF16 if score_dtype == "bf16" else hcsa.F32
        B, d, dev = st.B, st.d, st.device
        self.idx = torch.empty(B, Nq, topk, dtype=torch.int32, device=dev)
        self.out_csa = torch.empty(B, Nq, H, d, dtype=torch.float32, device=dev)
        self.lse_csa = torch.empty(B, Nq, H, dtype=torch.float32, device=dev)
        self.out_hca = torch.empty(B, Nq, H, d, dtype=torch.float32, device=dev)
        self.lse_hca = torch.empty(B, Nq, H, dtype=torch.float32, device=dev)
        self.scores = torch.empty(B * Nq, st.Nc, device=dev,
                                  dtype=torch.bfloat16 if score_dtype == "bf16" else torch.float32)
        self.ws_topk = hcsa.alloc_workspace(
            hcsa.topk_workspace_size(self.score_code, B, Nq, st.Nc, topk), dev)
        self.ws_itopk = hcsa.alloc_workspace(
            hcsa.index_topk_workspace_size(B, Nq, st.Nc, topk, self.score_code), dev)
        self.ws_attn = hcsa.alloc_workspace(
            hcsa.csa_hca_attn_workspace_size(B, Nq, H, d, topk, n_win, st.Nh), dev)
        self.ws_step = hcsa.alloc_workspace(
            hcsa.decode_step_workspace_size(B, Nq, st.Nc, topk, self.score_code, H, d, n_win,
                                            st.Nh), dev)

    def run_pool(self, pos0, stream=None):
        """Pool the blocks completed by the query tokens."""
        self.st.compress_range(pos0, pos0 + self.Nq, stream=stream)

    def run_index_scores(self, q_idx, w_idx, pos0, stream=None):
        """Indexer scores of every visible compressed entry (one kernel)."""
        st = self.st
        hcsa.csa_index_scores(q_idx, w_idx, st.Ic, st.Nc, R_CSA, pos0, self.scores,
                              k_scales=st.Ics, stream=stream, mx_fp8=self.mx_fp8)

    def _attend(self, q, pos0, stream):
        """CSA sparse attention and HCA dense attention of the query tokens (one call)."""
        st = self.st
        hcsa.csa_hca_attn(q, st.Kc, st.Vc, st.Nc, self.idx, st.K_raw, st.V_raw, 0, self.n_win,
                          R_CSA, st.Kh, st.Vh, st.Nh, R_HCA, pos0, self.scale, self.out_csa,
                          self.lse_csa, self.out_hca, self.lse_hca, workspace=self.ws_attn,
                          stream=stream)

    def run_select_attend(self, q, pos0, stream=None):
        st = self.st
        hcsa.topk(self.scores, st.B, self.Nq, st.Nc, R_CSA, pos0, self.topk, self.idx,
                  workspace=self.ws_topk, stream=stream)
        self._attend(q, pos0, stream)

    def run_index_topk(self, q_idx, w_idx, pos0, stream=None):
        """Indexer scores and top-k in one call with no score copy: for MXFP4 keys at
        decode the scores are never stored (floor, candidate scan, resolve)."""
        st = self.st
        hcsa.csa_index_topk(q_idx, w_idx, st.Ic, st.Nc, R_CSA, pos0, self.topk,
                            self.score_code, self.idx, k_scales=st.Ics,
                            workspace=self.ws_itopk, stream=stream, mx_fp8=self.mx_fp8)

    def run_pool_index_topk(self, q_idx, w_idx, pos0, stream=None):
        """Pooling of the blocks the query tokens complete, then indexer + top-k, as one
        call (for MXFP4 keys at decode the pooling shares the selection floors' launch)."""
        st = self.st
        hcsa.csa_pool_index_topk(st.pool_jobs(pos0, pos0 + self.Nq), q_idx, w_idx, st.Ic,
                                 st.Nc, R_CSA, pos0, self.topk, self.score_code, self.idx,
                                 k_scales=st.Ics, workspace=self.ws_itopk, stream=stream,
                                 mx_fp8=self.mx_fp8)

    def run_step(self, q, q_idx, w_idx, pos0, stream=None, noalloc=False):
        """The whole step (pooling of the completed blocks, indexer + top-k, CSA and HCA
        attention) as one call: for MXFP4 keys at one-token decode, four launches that run
        the HCA stream beside the floors and the resolves.  noalloc: the call that takes the
        library's fixed scratch instead of this step's workspace."""
        st = self.st
        args = (st.pool_jobs(pos0, pos0 + self.Nq), q_idx, w_idx, st.Ic, self.score_code,
                self.idx, q, st.Kc, st.Vc, st.Nc, self.topk, st.K_raw, st.V_raw, 0, self.n_win,
                R_CSA, st.Kh, st.Vh, st.Nh, R_HCA, pos0, self.scale, self.out_csa,
                self.lse_csa, self.out_hca, self.lse_hca)
        if noalloc:
            hcsa.decode_step_noalloc(*args, k_scales=st.Ics, stream=stream, mx_fp8=self.mx_fp8)
        else:
            hcsa.decode_step(*args, k_scales=st.Ics, workspace=self.ws_step, stream=stream,
                             mx_fp8=self.mx_fp8)
        return self.idx, (self.out_csa, self.lse_csa), (self.out_hca, self.lse_hca)

    def run_attend(self, q, pos0, stream=None):
        self._attend(q, pos0, stream)

    def run(self, q, q_idx, w_idx, pos0, append=True, scores_out=None, stream=None,
            marks=None, two_calls=False):
        """Full hot path for the query tokens at pos0..pos0+Nq-1: pool the blocks those
        tokens complete (append), indexer scores and top-k, CSA sparse attention and HCA
        attention.  By default (append, no score copy) one decode-step call; two_calls runs
        it as the pooling + indexer + top-k call and the attention call (same results).
        With scores_out the scores are written there and selected by a second call;
        without, the indexer + top-k never stores them for MXFP4 keys at decode.
        `marks`, if given, is called with a stage name before each stage and with "end"
        after the last (used to record timing events on the stream)."""
        st = self.st
        mark = marks or (lambda name: None)
        if scores_out is None and append and not two_calls and marks is None:
            return self.run_step(q, q_idx, w_idx, pos0, stream=stream)
        mark("pool_index_topk")
        if scores_out is None and append:
            self.run_pool_index_topk(q_idx, w_idx, pos0, stream=stream)
        elif scores_out is None:
            self.run_index_topk(q_idx, w_idx, pos0, stream=stream)
        else:
            if append:
                st.compress_range(pos0, pos0 + self.Nq, stream=stream)
            hcsa.csa_index_scores(q_idx, w_idx, st.Ic, st.Nc, R_CSA, pos0, scores_out,
                                  k_scales=st.Ics, stream=stream, mx_fp8=self.mx_fp8)
            hcsa.topk(scores_out, st.B, self.Nq, st.Nc, R_CSA, pos0, self.topk, self.idx,
                      workspace=self.ws_topk, stream=stream)
        mark("attention")
        self._attend(q, pos0, stream)
        mark("end")
        return self.idx, (self.out_csa, self.lse_csa), (self.out_hca, self.lse_hca)
