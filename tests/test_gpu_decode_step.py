"""One decode step as one call (hcsa_decode_step: floors, pooling and the first HCA splits
in one launch; the key scan; resolves, the remaining HCA splits and the CSA splits in one
launch; the merge) against the same step as two calls (hcsa_csa_pool_index_topk, then
hcsa_csa_hca_attn): pooled caches, selection and CSA attention equal bit for bit; HCA
attention, split finer in the four-launch form, within the bound that its bf16
probabilities allow between two split plans; and no wait of the back launch timed out.
Both paths are checked against the oracle in the end-to-end tests (the default step runs
through the single call)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_helpers import f64, pv_rounding_bound

pytestmark = pytest.mark.gpu

CASES = [
    # MXFP4 indexer at decode: the four-launch form
    dict(name="w5-b4-64k", cid=5, B=4, T=65536),
    dict(name="w5-b3-ragged-tail", cid=5, B=3, T=128 * 700),
    dict(name="w5-b32-full", cid=5, B=None, T=None),
    dict(name="w5-b1-1m", cid=5, B=1, T=1048576),
    # a front share of 0 and of all the safe splits
    dict(name="w5-front-none", cid=5, B=2, T=65536, front="0"),
    dict(name="w5-front-all", cid=5, B=2, T=65536, front="1000"),
    # other shapes take the two calls in turn inside the same call
    dict(name="cfg2-bf16-keys", cid=2, B=2, T=32768),
    dict(name="cfg1-fp32", cid=1, B=None, T=None),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_decode_step_equals_two_calls(gpu, case, monkeypatch):
    print(f"decode step {case['name']}", flush=True)
    if "front" in case:
        monkeypatch.setenv("HCSA_DECODE_HCA_FRONT", case["front"])
    cfg = W.CONFIGS[case["cid"]]
    if case["B"] is not None:
        cfg = W.small(cfg, B=case["B"], T=case["T"], pos0=case["T"] - 1)
    st, step, (q, qi, wi), om = W.build_case(cfg, gpu)
    from long_context_attention_26_amd.pipeline import DecodeStep
    step2 = DecodeStep(st.clone_caches(), cfg.Nq, cfg.H, cfg.H_I, cfg.topk, cfg.n_win,
                       cfg.score, cfg.scale)
    # junk in the outputs and the workspace: nothing may carry over
    for t in (step.idx, step.out_csa, step.lse_csa, step.out_hca, step.lse_hca):
        t.fill_(7)
    step.ws_step.fill_(0x5A)
    step.run_step(q, qi, wi, cfg.pos0)
    step2.run(q, qi, wi, cfg.pos0, two_calls=True)
    torch.cuda.synchronize()
    assert int(step.ws_step[:4].view(torch.int32).item()) == 0, "a selection wait timed out"
    for name in ("Kc", "Vc", "Kh", "Vh", "Ic", "Ics"):
        a, b = getattr(step.st, name), getattr(step2.st, name)
        if a is not None:
            assert torch.equal(a, b), f"{case['name']}: cache {name} differs"
    for a, b, what in ((step.idx, step2.idx, "idx"), (step.out_csa, step2.out_csa, "out_csa"),
                       (step.lse_csa, step2.lse_csa, "lse_csa")):
        assert torch.equal(a, b), f"{case['name']}: {what} differs"
    _hca_close(cfg, step, step2, q, case["name"])
    # a second step on the same workspace (the counters and flags were left set)
    out_h = step.out_hca.clone()
    step.run_step(q, qi, wi, cfg.pos0)
    torch.cuda.synchronize()
    assert int(step.ws_step[:4].view(torch.int32).item()) == 0
    assert torch.equal(step.idx, step2.idx) and torch.equal(step.out_csa, step2.out_csa)
    assert torch.equal(step.out_hca, out_h), "the step is not deterministic"


def _hca_close(cfg, step, step2, q, name):
    """HCA outputs of the two forms within the split-plan bound (exact when both forms split
    alike, as outside the four-launch form)."""
    a, b = f64(step.out_hca), f64(step2.out_hca)
    la, lb = f64(step.lse_hca), f64(step2.lse_hca)
    assert np.array_equal(np.isfinite(la), np.isfinite(lb))
    fin = np.isfinite(la)
    assert np.abs(la[fin] - lb[fin]).max(initial=0.0) <= 1e-5, f"{name}: HCA lse"
    Kh, Vh = f64(step.st.Kh), f64(step.st.Vh)
    qq = f64(q)
    for bb in range(cfg.B):
        n = O.visible_entries(cfg.pos0, Kh.shape[1], 128)
        bound = pv_rounding_bound(qq[bb, 0], Kh[bb, :n], Vh[bb, :n], cfg.scale)
        err = np.abs(a[bb, 0] - b[bb, 0])
        assert (err <= bound).all(), f"{name}: HCA sequence {bb}, worst {(err / bound).max()}"
