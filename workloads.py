"""Seeded synthetic inputs for the CSA/HCA attention path.

This module only draws random numbers and fixes shapes; it holds none of the method's
arithmetic, so both the HIP library's callers and the CPU oracle can take their inputs
from it.  All values are N(0,1) except the pooling logits (N(0,1)/sqrt(r)) and the
indexer head weights (|N(0,1)|/sqrt(H_I)).  bf16 tensors are drawn in fp32 and rounded
to nearest-even by torch.  Each (config, stream, sequence) has its own seed, so one
sequence of a large batch can be regenerated alone.
"""
from dataclasses import dataclass, replace

import numpy as np
import torch

SEED_BASE = 20260424

# stream ids
S_Q, S_KRAW, S_VRAW, S_IRAW, S_QIDX, S_WIDX = 0, 1, 2, 3, 4, 5
S_OMEGA = {"csa_k": 6, "csa_v": 7, "idx_k": 8, "hca_k": 9, "hca_v": 10}


@dataclass(frozen=True)
class Config:
    cid: int
    workload: str
    B: int            # sequences
    T: int            # context tokens per sequence (including the chunk for prefill)
    Nq: int           # query tokens per sequence
    pos0: int         # absolute position of query 0 (query i sits at pos0 + i)
    H: int            # query heads (one shared KV head)
    d: int            # head dim
    H_I: int          # indexer heads
    d_I: int          # indexer dim
    topk: int
    n_win: int
    kv: str           # "f32" | "bf16"
    idx: str          # storage of indexer keys: "f32" | "bf16" | "mxfp4"
    score: str        # "f32" | "bf16"
    r_csa: int = 4
    r_hca: int = 128

    @property
    def N_c(self):
        return self.T // self.r_csa

    @property
    def N_h(self):
        return self.T // self.r_hca

    @property
    def idx_raw(self):
        return "f32" if self.idx == "f32" else "bf16"

    @property
    def scale(self):
        return 1.0 / self.d ** 0.5


CONFIGS = {
    1: Config(1, "decode b1 ctx4096 fp32 H1 d64", B=1, T=4096, Nq=1, pos0=4095, H=1, d=64,
              H_I=1, d_I=32, topk=64, n_win=128, kv="f32", idx="f32", score="f32"),
    2: Config(2, "decode b8 ctx131072 bf16 H16 d128", B=8, T=131072, Nq=1, pos0=131071, H=16,
              d=128, H_I=4, d_I=64, topk=512, n_win=128, kv="bf16", idx="bf16", score="bf16"),
    3: Config(3, "decode b1 ctx1048576 bf16 H16 d128", B=1, T=1048576, Nq=1, pos0=1048575,
              H=16, d=128, H_I=4, d_I=64, topk=1024, n_win=128, kv="bf16", idx="bf16",
              score="bf16"),
    4: Config(4, "prefill chunk4096 on 262144 cached bf16 H16 d128", B=1, T=262144 + 4096,
              Nq=4096, pos0=262144, H=16, d=128, H_I=4, d_I=64, topk=512, n_win=128,
              kv="bf16", idx="bf16", score="bf16"),
    5: Config(5, "decode b32 ctx1048576 bf16 H16 d128 mxfp4 indexer", B=32, T=1048576, Nq=1,
              pos0=1048575, H=16, d=128, H_I=4, d_I=64, topk=1024, n_win=128, kv="bf16",
              idx="mxfp4", score="bf16"),
}


def small(cfg, **kw):
    """A copy of cfg with some fields replaced (used for reduced-size test cases)."""
    return replace(cfg, **kw)


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(cid, stream, b, device):
    g = torch.Generator(device=device)
    seq = np.random.SeedSequence([SEED_BASE, cid, stream, b])
    g.manual_seed(int(seq.generate_state(1, np.uint64)[0]) & ((1 << 63) - 1))
    return g


def normal(shape, cid, stream, b=0, device="cpu", dtype="f32", std=1.0, absolute=False):
    """N(0, std^2) draws (|.| if absolute) in fp32, then cast to dtype."""
    x = torch.randn(shape, generator=_gen(cid, stream, b, device), device=device,
                    dtype=torch.float32)
    if absolute:
        x = x.abs()
    if std != 1.0:
        x = x * std
    return x.to(torch_dtype(dtype))


def raw_sequence(cfg, b, device="cpu", rows=None):
    """Raw (uncompressed) K, V and indexer-key rows of sequence b: [T, d], [T, d], [T, d_I]."""
    T = cfg.T if rows is None else rows
    K = normal((T, cfg.d), cfg.cid, S_KRAW, b, device, cfg.kv)
    V = normal((T, cfg.d), cfg.cid, S_VRAW, b, device, cfg.kv)
    I = normal((T, cfg.d_I), cfg.cid, S_IRAW, b, device, cfg.idx_raw)
    return K, V, I


def queries(cfg, device="cpu"):
    """q [B, Nq, H, d], indexer queries [B, Nq, H_I, d_I], indexer weights [B, Nq, H_I]."""
    q = normal((cfg.B, cfg.Nq, cfg.H, cfg.d), cfg.cid, S_Q, 0, device, cfg.kv)
    qi = normal((cfg.B, cfg.Nq, cfg.H_I, cfg.d_I), cfg.cid, S_QIDX, 0, device, cfg.idx_raw)
    wi = normal((cfg.B, cfg.Nq, cfg.H_I), cfg.cid, S_WIDX, 0, device, "f32",
                std=cfg.H_I ** -0.5, absolute=True)
    return q, qi, wi


def pool_logits(cfg, device="cpu"):
    """Per-position pooling logits omega for the five compressed streams (fp32)."""
    out = {}
    for name, stream in S_OMEGA.items():
        r = cfg.r_hca if name.startswith("hca") else cfg.r_csa
        out[name] = normal((r,), cfg.cid, stream, 0, device, "f32", std=r ** -0.5)
    return out


def build_case(cfg, device, seqs=None):
    """Raw tokens, pooled caches (every block completed before pos0) and query inputs of
    `cfg` on `device`; returns (state, step, (q, q_idx, w_idx), omegas).  The step's own
    run() pools the blocks completed by the query tokens themselves.  `seqs` restricts
    the batch to a list of sequence ids (each keeps its own seed)."""
    from long_context_attention_26_amd.pipeline import DecodeStep, HybridAttentionState

    seqs = list(range(cfg.B)) if seqs is None else list(seqs)
    B = len(seqs)
    om = pool_logits(cfg, device)
    st = HybridAttentionState(B, cfg.T, cfg.d, cfg.d_I, torch_dtype(cfg.kv), cfg.idx, device, om)
    K = torch.empty(B, cfg.T, cfg.d, dtype=torch_dtype(cfg.kv), device=device)
    V = torch.empty_like(K)
    I = torch.empty(B, cfg.T, cfg.d_I, dtype=torch_dtype(cfg.idx_raw), device=device)
    for i, b in enumerate(seqs):
        K[i], V[i], I[i] = raw_sequence(cfg, b, device)
    st.attach_raw(K, V, I)
    st.compress_range(0, cfg.pos0)
    q, qi, wi = queries(cfg, device)
    q, qi, wi = q[seqs].contiguous(), qi[seqs].contiguous(), wi[seqs].contiguous()
    step = DecodeStep(st, cfg.Nq, cfg.H, cfg.H_I, cfg.topk, cfg.n_win, cfg.score, cfg.scale)
    return st, step, (q, qi, wi), om
