#!/usr/bin/env python3
"""Decode throughput of the CSA + HCA hybrid compressed attention hot path on one MI355X.

One step = one decode token of every sequence of the batch through the whole path:
pooling of the blocks that token completes (CSA K/V/indexer keys, HCA K/V), indexer
scores, top-k, CSA sparse attention (selected entries + 128-token window) and HCA dense
attention.  Inputs are seeded synthetic tensors already resident in HBM.  The pooled
caches are rotated over several copies so that the 256 MB Infinity Cache cannot hold the
working set of consecutive steps (HBM-cold steps).

Prints one JSON line.  --gpus above 1 is not supported (single-GPU build).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "1M-ctx compressed-attn decode queries/s + achieved HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
MALL_BYTES = 256 << 20


def _visible(cfg, ratio):
    """Entries of one compressed stream seen by each query token of a step."""
    N = cfg.T // ratio
    return [min(N, (cfg.pos0 + i + 1) // ratio) for i in range(cfg.Nq)]


def step_bytes(cfg):
    """Algorithmic HBM bytes of one step.  Decode (one query token per sequence): per
    sequence the indexer-key scan, the gathered top-k + window K/V rows, the HCA entries,
    the pooling reads of the completed blocks, q and outputs.  Prefill (a chunk of query
    tokens per sequence): every cache row is needed once per chunk, so the same items count
    the caches once (the CSA rows gathered at most once each), the chunk's raw tokens for
    the window and pooling, and q and outputs per token."""
    kv = 4 if cfg.kv == "f32" else 2
    if cfg.idx == "mxfp4":
        key = cfg.d_I // 2 + cfg.d_I // 32
    else:
        key = cfg.d_I * (4 if cfg.idx == "f32" else 2)
    if cfg.Nq == 1:
        per = {
            "index_scan": cfg.N_c * key,
            "gather": (cfg.topk + cfg.n_win) * 2 * cfg.d * kv,
            "hca": cfg.N_h * 2 * cfg.d * kv,
            "pool": (2 * 4 * cfg.d + 4 * cfg.d_I) * kv + 2 * 128 * cfg.d * kv,
            "q_out": cfg.H * cfg.d * (kv + 2 * 4),
        }
    else:
        per = {
            "index_scan": cfg.N_c * key,
            "gather": min(cfg.N_c, cfg.Nq * cfg.topk) * 2 * cfg.d * kv
                      + (cfg.Nq + cfg.n_win) * 2 * cfg.d * kv,
            "hca": cfg.N_h * 2 * cfg.d * kv,
            "pool": cfg.Nq * (2 * cfg.d + cfg.d_I + 2 * cfg.d) * kv,
            "q_out": cfg.Nq * cfg.H * cfg.d * (kv + 2 * 4),
        }
    return {k: v * cfg.B for k, v in per.items()}


def step_flops(cfg):
    """Algorithmic floating-point operations of one step (multiply-add = 2): indexer dot
    products over the visible compressed entries of every query token and indexer head,
    CSA attention over the selected entries plus the window, HCA attention over every
    visible entry (QK^T and PV, 4 per key per channel per head)."""
    nv_c, nv_h = _visible(cfg, cfg.r_csa), _visible(cfg, cfg.r_hca)
    idx = sum(nv_c) * cfg.H_I * cfg.d_I * 2
    csa = sum(min(cfg.topk, n) + min(cfg.n_win, cfg.pos0 + i + 1)
              for i, n in enumerate(nv_c)) * cfg.H * cfg.d * 4
    hca = sum(nv_h) * cfg.H * cfg.d * 4
    return {"index": idx * cfg.B, "csa": csa * cfg.B, "hca": hca * cfg.B}


def index_scan_bytes(cfg):
    return step_bytes(cfg)["index_scan"]


def measured_traffic(cfg, mx_fp8=False):
    """HBM bytes per indexer launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary (scaled by a copy kernel of known size), if it covers this workload and the
    kernel's source text is unchanged since it was taken; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "index_scores_mx_mfma_decode_b32_1m_counters.json")
    if cfg.cid != 5 or mx_fp8 or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    csrc = os.path.join(ROOT, "long_context_attention_26_amd", "csrc")
    src = "".join(open(os.path.join(csrc, f)).read() for f in ("mx_dev.h", "mx_scan.h"))
    if hashlib.sha256(src.encode()).hexdigest() != rec.get("kernel_text_sha256"):
        return None
    return int(round(rec["traffic_bytes"]))


def _host_cpus():
    """CPUs this process may run on, and the host's CPU model name."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(cfg, st, om, q, qi, wi, seconds, gpu_idx=None):
    """The CPU oracle on sequence 0: its own pooled caches are built untimed from the raw
    tokens, then whole decode queries (pooling of the completed blocks, indexer, top-k,
    CSA and HCA attention) are timed until `seconds` of work, with the BLAS thread pool as
    configured and then with one thread.  With the GPU's selection of sequence 0 it also
    reports the recall of that selection against the exact fp32 top-k of the unquantized
    (bf16-stored) indexer queries and keys."""
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits

    f = lambda t: t.float().cpu().double().numpy()
    K, V, I = f(st.K_raw[0]), f(st.V_raw[0]), f(st.I_raw[0])
    omd = {k: f(v) for k, v in om.items()}
    p = cfg.pos0
    # caches of every block completed before p (untimed); the last entry of each stream
    # is pooled inside the timed query, as in the GPU step
    Kc = O.round_to(O.compress(K[: p + 1], omd["csa_k"], 4), cfg.kv)
    Vc = O.round_to(O.compress(V[: p + 1], omd["csa_v"], 4), cfg.kv)
    Kh = O.round_to(O.compress(K[: p + 1], omd["hca_k"], 128), cfg.kv)
    Vh = O.round_to(O.compress(V[: p + 1], omd["hca_v"], 128), cfg.kv)
    Ic_exact = O.compress(I[: p + 1], omd["idx_k"], 4)
    Ic = O.mxfp4_roundtrip(Ic_exact) if cfg.idx == "mxfp4" else O.round_to(Ic_exact, cfg.idx)
    qv, qiv, wiv = f(q[0, 0]), f(qi[0, 0]), f(wi[0, 0])
    c0 = 4 * (Kc.shape[0] - 1)                 # tokens of the last completed entries
    h0 = 128 * (Kh.shape[0] - 1)

    def query():
        Kc[-1] = O.round_to(O.compress(K[c0: c0 + 4], omd["csa_k"], 4), cfg.kv)[0]
        Vc[-1] = O.round_to(O.compress(V[c0: c0 + 4], omd["csa_v"], 4), cfg.kv)[0]
        ic = O.compress(I[c0: c0 + 4], omd["idx_k"], 4)
        qq = qiv
        if cfg.idx == "mxfp4":
            Ic[-1] = O.mxfp4_roundtrip(ic)[0]
            qq = O.mxfp4_roundtrip(qiv)
        else:
            Ic[-1] = O.round_to(ic, cfg.idx)[0]
        Kh[-1] = O.round_to(O.compress(K[h0: h0 + 128], omd["hca_k"], 128), cfg.kv)[0]
        Vh[-1] = O.round_to(O.compress(V[h0: h0 + 128], omd["hca_v"], 128), cfg.kv)[0]
        return O.decode_query(qv, qq, wiv, Kc, Vc, Ic, K, V, 0, Kh, Vh, p, cfg.topk, cfg.n_win,
                              cfg.scale, cfg.score)

    def rate(secs):
        query()  # warm-up
        n, t0 = 0, time.perf_counter()
        while True:
            query()
            n += 1
            el = time.perf_counter() - t0
            if el >= secs:
                return n / el, n, el

    value, n, el = rate(seconds)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    with threadpool_limits(limits=1):
        one, n1, el1 = rate(seconds / 2)
    host, model = _host_cpus()
    what = "decode queries" if cfg.Nq == 1 else "prefill query tokens (the chunk's first)"
    unit = "decode queries/s" if cfg.Nq == 1 else "prefill query tokens/s"
    out = {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
           "sample": f"{n} {what} of sequence 0 (p={p}, full context) through the "
                     f"float64 numpy oracle, {el:.1f} s ({threads} BLAS threads); caches "
                     f"pooled untimed",
           "single_core_value": one, "single_core_sample": f"{n1} queries, {el1:.1f} s",
           "host_cpus": host, "cpu_model": model}
    if gpu_idx is not None:
        nv = O.visible_entries(p, Kc.shape[0], 4)
        ref = O.select_topk(O.index_scores(O.round_bf16(qiv), wiv, O.round_bf16(Ic_exact), nv,
                                           "f32"), nv, cfg.topk)
        g = set(int(j) for j in gpu_idx if j >= 0)
        r = set(int(j) for j in ref if j >= 0)
        out["recall"] = {"value": len(g & r) / max(1, len(r)), "sequence": 0,
                         "reference": "exact fp32 top-k of the bf16-stored indexer query and "
                                      "keys (no MXFP4 rounding)",
                         "context": "the pages quote 99.7 % on real model data"}
    return out


def selector_ratio(cfg, stp, q_idx, w_idx, dev, reps=20):
    """Top-k selector on the same indexer scores stored as fp32 and as bf16 (the pages'
    FP32 -> BF16 index-score change for the selector): the selector call's average time
    for each and their ratio."""
    import torch
    from long_context_attention_26_amd import hcsa
    st = stp.st
    rows, N = cfg.B * cfg.Nq, st.Nc
    res = {}
    for name, code, dt in (("fp32", hcsa.F32, torch.float32), ("bf16", hcsa.BF16, torch.bfloat16)):
        sc = torch.empty(rows, N, dtype=dt, device=dev)
        hcsa.csa_index_scores(q_idx, w_idx, st.Ic, N, 4, cfg.pos0, sc, k_scales=st.Ics)
        idx = torch.empty(rows, cfg.topk, dtype=torch.int32, device=dev)
        ws = hcsa.alloc_workspace(hcsa.topk_workspace_size(code, cfg.B, cfg.Nq, N, cfg.topk), dev)
        for _ in range(3):
            hcsa.topk(sc, cfg.B, cfg.Nq, N, 4, cfg.pos0, cfg.topk, idx, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            hcsa.topk(sc, cfg.B, cfg.Nq, N, 4, cfg.pos0, cfg.topk, idx, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        res[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
        del sc
    res["speedup_bf16_over_fp32"] = round(res["fp32_us"] / res["bf16_us"], 3)
    res["note"] = (f"{rows} row(s) of {N} scores, k {cfg.topk}; back-to-back calls (scores "
                   "partly cache-resident); context: the pages quote 2x")
    return res


def copy_calibration():
    """Three launches of a plain copy of exactly 2 GiB (read 2 GiB, write 2 GiB): what the
    FETCH_SIZE / WRITE_SIZE counters read for it converts their units into bytes."""
    import torch
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def train_backward(args):
    """--train: the attention part of one training step at the 64K stage of the length
    curriculum (one sequence of 65 536 tokens, every token a query; CSA top-1024 + window
    128, HCA, 16 heads x 128, bf16).  The selection (indexer + top-k over all 65 536 rows)
    and the forward run untimed first; the timed step is the backward: zeroing the
    gradient buffers, CSA attention backward, HCA attention backward and the pooling
    backward of the four pooled K/V streams into the raw-token gradients and the pooling
    logits.  The forward (CSA + HCA) is timed beside it for the ratio.  Prints one JSON
    line."""
    import torch
    import workloads as W
    from long_context_attention_26_amd import hcsa

    T, Hh, d, H_I, d_I, k, w = 65536, 16, 128, 4, 64, 1024, 128
    cfg = W.Config(0, "train b1 ctx65536 bf16 H16 d128 topk1024", B=1, T=T, Nq=T, pos0=0,
                   H=Hh, d=d, H_I=H_I, d_I=d_I, topk=k, n_win=w, kv="bf16", idx="bf16",
                   score="bf16")
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    K, V, I = (x.to(dev).unsqueeze(0) for x in W.raw_sequence(cfg, 0))
    om = W.pool_logits(cfg, dev)
    q, qi, wi = (x.to(dev) for x in W.queries(cfg))
    Nc, Nh = T // 4, T // 128
    Kc, Vc, Ic = (torch.empty(1, Nc, D, dtype=bf, device=dev) for D in (d, d, d_I))
    Kh, Vh = (torch.empty(1, Nh, d, dtype=bf, device=dev) for _ in range(2))
    hcsa.compress_kv_batched([hcsa.pool_job(K, om["csa_k"], 4, Kc), hcsa.pool_job(V, om["csa_v"], 4, Vc),
                              hcsa.pool_job(I, om["idx_k"], 4, Ic), hcsa.pool_job(K, om["hca_k"], 128, Kh),
                              hcsa.pool_job(V, om["hca_v"], 128, Vh)], 1)
    # a call takes at most 65 535 query rows: the sequence's tokens go in two halves
    HALF = T // 2
    halves = [(h0, slice(h0, h0 + HALF)) for h0 in (0, HALF)]
    idx = torch.empty(1, T, k, dtype=torch.int32, device=dev)
    for h0, sl in halves:
        hcsa.csa_index_topk(qi[:, sl], wi[:, sl], Ic, Nc, 4, h0, k, hcsa.BF16, idx[:, sl])
    scale = cfg.scale
    oc, oh = (torch.empty(1, T, Hh, d, device=dev) for _ in range(2))
    lc, lh = (torch.empty(1, T, Hh, device=dev) for _ in range(2))
    ws_c = hcsa.alloc_workspace(hcsa.csa_attn_workspace_size(1, HALF, Hh, d, k, w), dev)
    ws_h = hcsa.alloc_workspace(hcsa.hca_attn_workspace_size(1, HALF, Hh, d, Nh), dev)

    def forward():
        for h0, sl in halves:
            hcsa.csa_sparse_attn(q[:, sl], Kc, Vc, Nc, idx[:, sl], K, V, 0, w, 4, h0, scale,
                                 oc[:, sl], lc[:, sl], workspace=ws_c)
            hcsa.hca_dense_attn(q[:, sl], Kh, Vh, Nh, 128, h0, scale, oh[:, sl], lh[:, sl],
                                workspace=ws_h)

    forward()
    g = torch.Generator(device=dev).manual_seed(7)
    doc = torch.randn(1, T, Hh, d, device=dev, generator=g)
    doh = torch.randn(1, T, Hh, d, device=dev, generator=g)
    dqc, dqh = torch.empty_like(doc), torch.empty_like(doh)
    grads = {n: torch.zeros(1, r_, d, device=dev) for n, r_ in
             (("Kc", Nc), ("Vc", Nc), ("Kh", Nh), ("Vh", Nh), ("K", T), ("V", T))}
    dom = {n: torch.zeros(r_, device=dev) for n, r_ in
           (("csa_k", 4), ("csa_v", 4), ("hca_k", 128), ("hca_v", 128))}
    ws_p = hcsa.alloc_workspace(hcsa.lib.hcsa_compress_kv_bwd_workspace_size(1, T, 128), dev)
    ws_hb = hcsa.alloc_workspace(
        hcsa.lib.hcsa_hca_dense_attn_bwd_workspace_size(1, HALF, Hh, d, hcsa.BF16), dev)
    ws_cb = hcsa.alloc_workspace(
        hcsa.lib.hcsa_csa_sparse_attn_bwd_workspace_size(1, HALF, Hh, d, hcsa.BF16, Nc, k),
        dev)

    stages = ["zero", "csa_bwd", "hca_bwd", "pool_bwd"]

    def backward(ev=None):
        mark = (lambda i: ev[i].record()) if ev else (lambda i: None)
        mark(0)
        for t in grads.values():
            t.zero_()
        for t in dom.values():
            t.zero_()
        mark(1)
        for h0, sl in halves:
            hcsa.csa_sparse_attn_bwd(q[:, sl], Kc, Vc, Nc, idx[:, sl], K, V, 0, w, 4, h0, scale,
                                     oc[:, sl], lc[:, sl], doc[:, sl], dqc[:, sl], grads["Kc"],
                                     grads["Vc"], grads["K"], grads["V"], workspace=ws_cb)
        mark(2)
        for h0, sl in halves:
            hcsa.hca_dense_attn_bwd(q[:, sl], Kh, Vh, Nh, 128, h0, scale, oh[:, sl], lh[:, sl],
                                    doh[:, sl], dqh[:, sl], grads["Kh"], grads["Vh"],
                                    workspace=ws_hb)
        mark(3)
        for x, n, r_, gy, gx in ((K, "csa_k", 4, "Kc", "K"), (V, "csa_v", 4, "Vc", "V"),
                                 (K, "hca_k", 128, "Kh", "K"), (V, "hca_v", 128, "Vh", "V")):
            hcsa.compress_kv_bwd(x, om[n], r_, grads[gy], grads[gx], dom[n], workspace=ws_p)
        mark(4)

    nvtx = torch.cuda.nvtx                       # roctx ranges (rocprofv3 --marker-trace)
    nvtx.range_push("backward warmup")
    for _ in range(args.warmup):
        backward()
    torch.cuda.synchronize()
    nvtx.range_pop()
    evs = []
    nvtx.range_push("backward timed steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        backward(e)
        evs.append(e)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / args.steps
    nvtx.range_pop()
    br = {s_: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / len(evs) for j, s_ in enumerate(stages)}
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(args.steps):
        forward()
    f1.record()
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / args.steps

    # (query, key) pairs of the CSA backward: selected entries plus window of every token
    pairs = sum(min(k, (p + 1) // 4) + min(w, p + 1) for p in range(T))
    flops = pairs * 5 * 2 * Hh * d          # q.k, dout.v, dk, dv, dq: H*d multiply-adds each
    achieved = flops / (br["csa_bwd"] * 1e-3) / 1e12   # bf16 products on the matrix cores
    out = {
        "metric": "training attention backward tokens/s (CSA + HCA + pooling, 64K stage)",
        "value": round(T / el, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(el * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens and output gradients)",
        "config": {"workload": cfg.workload, "context": T, "queries": T, "heads": Hh,
                   "head_dim": d, "topk": k, "n_win": w},
        "breakdown_ms": {k_: round(v, 3) for k_, v in br.items()},
        "forward_ms": round(fwd_ms, 3),
        "roofline": {"kernel": "CSA attention backward (sort, dq pass, key-major selected "
                               "entries and window rows; 2 calls)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "flops_per_step": flops,
                     "note": "algorithmic flops over the csa_bwd stage time; the dq pass "
                             "gathers key rows query-major, the selected entries' dK/dV run as "
                             "dense products over 128-entry tiles (about 8 % of whose "
                             "(token, entry) cells are selected)"},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5,
                    help="workload id (1..5); default 5: decode, batch 32, 1M-token context")
    ap.add_argument("--rotate", type=int, default=0, help="cache copies (0 = enough to defeat the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mx-fp8", action="store_true",
                    help="MXFP4 indexer keys (workload 5): scan them on FP8 operands (codes "
                         "widened to e4m3) instead of FP4 ones")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 2 GiB device-to-device copy 3 times (the known-size "
                         "kernel that scales the HBM byte counters)")
    ap.add_argument("--train", action="store_true",
                    help="time the training backward (CSA + HCA attention and pooling) at "
                         "one 65 536-token sequence instead of the decode step")
    args = ap.parse_args()
    if args.train:
        if args.gpus != 1:
            sys.exit("bench.py: the benchmark runs on one GPU only (--gpus 1)")
        train_backward(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); how the path would shard over several GPUs is "
              "described, not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W

    cfg = W.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    st, step0, (q, qi, wi), om = W.build_case(cfg, dev)
    sb = step_bytes(cfg)
    total_bytes = sum(sb.values())
    R = args.rotate or max(2, math.ceil(2 * MALL_BYTES / total_bytes))
    from long_context_attention_26_amd import hcsa
    from long_context_attention_26_amd.pipeline import DecodeStep
    steps = [step0] + [DecodeStep(st.clone_caches(), cfg.Nq, cfg.H, cfg.H_I, cfg.topk, cfg.n_win,
                                  cfg.score, cfg.scale) for _ in range(R - 1)]
    if args.mx_fp8:
        if cfg.idx != "mxfp4":
            sys.exit("bench.py: --mx-fp8 needs a workload with MXFP4 indexer keys (5)")
        for stp in steps:
            stp.mx_fp8 = True
    torch.cuda.synchronize()

    # Each copy's step (one decode-step call) is captured as one HIP graph.  Every SAMPLE-th
    # timed step runs the call directly, its key scan recording dispatch-level events (the
    # kernel's own duration, for the roofline), with events around the whole call.  The
    # SAMPLE - 1 steps between two sampled ones replay one graph that chains them (each on
    # its own cache copy, every kernel of every step executed), as a model's per-token graph
    # chains its layers: the host's graph-launch latency, several microseconds per launch,
    # then falls on one step in SAMPLE instead of every step.  Timed step i runs on copy
    # (warmup + i) mod R, so the first timed step does not read the copy the last warm-up
    # step has just streamed (part of it would still sit in the Infinity Cache).
    SAMPLE = 16
    full = []
    cap_stream = torch.cuda.Stream()
    for stp in steps:
        for _ in range(2):                      # run once eagerly before capture
            stp.run_step(q, qi, wi, cfg.pos0)
        torch.cuda.synchronize()
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap_stream):
            g_all.capture_begin()
            stp.run_step(q, qi, wi, cfg.pos0)
            g_all.capture_end()
        full.append(g_all)
    torch.cuda.synchronize()
    chain = []                                  # chain[c]: SAMPLE - 1 steps from copy c on
    for c in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap_stream):
            g.capture_begin()
            for j in range(SAMPLE - 1):
                steps[(c + j) % R].run_step(q, qi, wi, cfg.pos0)
            g.capture_end()
        chain.append(g)
    torch.cuda.synchronize()

    ev, kev = [], []
    base = args.warmup

    def one_step(c, sampled):
        if sampled:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e[0].record()
            hcsa.time_next_indexer(k0, k1)
            steps[c].run_step(q, qi, wi, cfg.pos0)
            e[1].record()
            ev.append(e)
            kev.append((k0, k1))
        else:
            full[c].replay()

    nvtx = torch.cuda.nvtx                       # roctx ranges (rocprofv3 --marker-trace)
    nvtx.range_push("decode warmup")
    for i in range(args.warmup):
        one_step(i % R, False)
    torch.cuda.synchronize()
    nvtx.range_pop()
    assert args.steps == 0 or (base % R) != ((args.warmup - 1) % R) or R == 1
    nvtx.range_push("decode timed steps")
    t0 = time.perf_counter()
    i = 0
    while i < args.steps:
        if i % SAMPLE == 1 and i + SAMPLE - 1 <= args.steps:
            chain[(base + i) % R].replay()       # steps i .. i + SAMPLE - 2
            i += SAMPLE - 1
        else:
            one_step((base + i) % R, i % SAMPLE == 0)
            i += 1
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    nvtx.range_pop()
    ms = el / args.steps * 1e3
    qps = cfg.B * cfg.Nq / (el / args.steps)

    # durations from the events recorded on the launch stream
    idx_us = sum(a.elapsed_time(b) for a, b in kev) * 1e3 / len(kev)
    br = {"step_call": sum(e[0].elapsed_time(e[1]) for e in ev) * 1e3 / len(ev),
          "key_scan": idx_us}
    flops = step_flops(cfg)
    if cfg.Nq == 1:
        # decode: the indexer streams every compressed key once per query
        achieved = index_scan_bytes(cfg) / (idx_us * 1e-6) / 1e9
        kname = ("index_scores_mx_mfma_kernel (MXFP4 key scan writing candidate lists; no "
                 "score array)" if cfg.idx == "mxfp4" else
                 "index_scores_kernel (key scan writing the score array)")
        roof = {"kernel": kname, "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(cfg, args.mx_fp8),
                "bytes_per_launch": index_scan_bytes(cfg)}
    else:
        # prefill: one launch scores every query token of the chunk against every visible
        # key, a bf16 matrix-core contraction
        achieved = flops["index"] / (idx_us * 1e-6) / 1e12
        roof = {"kernel": "index_scores (lightning-indexer MFMA GEMM)", "bound": "mfma",
                "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None, "flops_per_launch": flops["index"]}
    roof.update({"avg_launch_us": round(idx_us, 3),
                 "timing": "dispatch-recorded start/stop events on the launch stream"})
    unit = "decode queries/s" if cfg.Nq == 1 else "prefill query tokens/s"
    out = {
        "metric": METRIC,
        "value": round(qps, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.kv == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens, random pooling logits and indexer weights)",
        "config": {"workload": cfg.workload, "batch": cfg.B, "context": cfg.T, "heads": cfg.H,
                   "head_dim": cfg.d,
                   "indexer": f"{cfg.H_I}x{cfg.d_I} {cfg.idx}"
                              + (" on fp8 operands" if args.mx_fp8 else ""),
                   "scores": cfg.score, "topk": cfg.topk, "n_win": cfg.n_win,
                   "cache_copies_rotated": R},
        "step_hbm_gbps": round(total_bytes / (el / args.steps) / 1e9, 1),
        "step_hbm_frac": round(total_bytes / (el / args.steps) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_bytes": total_bytes,
        "step_tflops": round(sum(flops.values()) / (el / args.steps) / 1e12, 2),
        "breakdown_us": {k: round(v, 2) for k, v in br.items()},
        "breakdown_note": f"sampled every {SAMPLE}th step ({len(ev)} samples): the decode-step "
                          "call launched directly (host launch included) and its key scan "
                          "kernel alone; the steps between samples replay one graph of "
                          f"{SAMPLE - 1} chained steps",
        "roofline": roof,
    }
    if cfg.Nq == 1 and cfg.score == "bf16":
        out["selector_fp32_vs_bf16"] = selector_ratio(cfg, steps[0], qi, wi, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, st, om, q, qi, wi, args.cpu_seconds,
                                           gpu_idx=step0.idx[0, 0].cpu().numpy())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
