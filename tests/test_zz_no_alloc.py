"""moe_plan_noalloc (the plan with its scratch in a static per-GPU array) against moe_plan with a
caller-owned workspace, through the C ABI: counts, plan blob and status bit for bit, on two
calls in a row, the second with a smaller routing (the static scratch still holds the first
call's partial histograms), and a third back at the large size.  Both are also checked
against the oracle's plan."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import log, mod, poisoned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mod()


def _plan_both(m, d, idx):
    """(counts, blob, status) of moe_plan_noalloc, then of moe_plan, on the same routing."""
    lib = m.library()
    md = m.dims(d.R, d.S, d.K, d.E, d.B)
    topk = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for noalloc in (True, False):
        counts = poisoned((d.R, d.E), torch.int32)
        plan = poisoned((m.plan_words(md),), torch.int32)
        status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        if noalloc:
            rc = lib.moe_plan_noalloc(ctypes.byref(md), P(topk), P(counts), P(plan), P(status),
                                      stream)
        else:
            ws = torch.empty(m.plan_workspace_bytes(md), dtype=torch.uint8, device="cuda")
            rc = lib.moe_plan(ctypes.byref(md), P(topk), P(counts), P(plan), P(status), P(ws),
                              ctypes.c_size_t(ws.numel()), stream)
        assert rc == m.MOE_OK, lib.moe_status_string(rc)
        torch.cuda.synchronize()
        out.append((counts.cpu().numpy(), plan.cpu().numpy(), int(status.item())))
    return out


def test_plan_noalloc_matches_plan_two_sizes():
    m = mod()
    cases = [("skew8_large_fwdbwd", 8.0), ("tiny_f32", None), ("skew1_large", 1.0)]
    for name, target in cases:
        wl = synth.WORKLOADS[name]
        d = wl.dims
        zipf = synth.zipf_for(wl, target) if target is not None else wl.zipf_s
        idx, _ = synth.routing(d, zipf, wl.base_seed)
        log(f"plan_noalloc {name} R{d.R} S{d.S} K{d.K} E{d.E} B{d.B} target {target}")
        (c0, b0, s0), (c1, b1, s1) = _plan_both(m, d, idx)
        assert (c0 == c1).all(), "counts"
        assert (b0 == b1).all(), f"plan blob differs at {np.nonzero(b0 != b1)[0][:10]}"
        assert s0 == s1
        pl = oracle.plan(idx, d.E, d.B)
        assert (c0 == pl.counts).all() and (b0 == pl.to_blob()).all() and s0 == pl.status
