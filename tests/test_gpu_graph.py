"""One layer step captured in a HIP graph and replayed: every replay reproduces the eager
step bit for bit.

The library makes no allocation, memset, host synchronisation or host read inside its entry
points, so a whole forward + backward step (plan, layout, prefetch, permute, grouped GEMMs,
combine, the backward kernels and the fold) can be captured once and replayed; also with the
permute fused into the up GEMM and the plan on the library's static scratch (moe_plan_noalloc,
whose device address is looked up before capture, on the eager step).  The test replays the
graph several times with eager steps and eager work in between and compares every output of
every replay with the eager step's.  A second test checks that the step with its backward's
second stream (event fork and join) matches the step in one stream bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(L):
    t = {"plan": L.plan, "cu": L.cu, "dest": L.dest, "src": L.src, "xp": L.xp, "z": L.z,
         "y": L.y, "out": L.out, "dy": L.dy, "dz": L.dz, "dxp": L.dxp, "dx": L.dx,
         "dtopk_w": L.dtopk_w, "dw_up": L.dw_up, "dw_down": L.dw_down, "w_up": L.w_up}
    if L.activation == "swiglu":
        t["h"], t["dh"] = L.hpre, L.dh
    return {k: v.clone() for k, v in t.items() if v is not None}


# (activation, permute fused into the up GEMM, plan on the library's static scratch)
CASES = [("identity", False, False), ("swiglu", False, False), ("identity", True, True)]


@pytest.mark.parametrize("activation,fused,noalloc", CASES)
def test_layer_step_graph_replay(activation, fused, noalloc):
    from balanced_token_dispatch_amd.layer import LayerStep, Shape
    d = synth.Dims(R=8, S=512, K=4, E=32, B=4, H=256, Hp=192)
    idx, w = synth.routing(d, 1.0, 21)
    L = LayerStep(Shape(d.R, d.S, d.K, d.E, d.B, d.H, d.Hp), rank=1, activation=activation,
                  fused_gather=fused, plan_noalloc=noalloc)
    synth.fill_normal_(L.x_all, 1.0, 211)
    synth.fill_normal_(L.w_up, 0.05, 212)
    synth.fill_normal_(L.w_down, 0.05, 213)
    synth.fill_normal_(L.y_all, 1.0, 214)
    synth.fill_normal_(L.dout_all, 1.0, 215)
    synth.fill_normal_(L.dxp_all, 1.0, 216)
    L.topk_idx.copy_(torch.from_numpy(idx))
    L.topk_w.copy_(torch.from_numpy(w))

    def step():
        L.dw_up.zero_()   # a fill kernel, not a memset node
        L.dw_down.zero_()
        L.step()

    step()
    torch.cuda.synchronize()
    ref = _outputs(L)
    assert int(L.status.item()) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: overwrite every output buffer, then replay
        for name in ("counts", "plan", "cu", "dest", "src", "xp", "z", "y", "out", "dy", "dz",
                     "dxp", "dx", "dtopk_w", "dw_up", "dw_down", "hpre", "dh"):
            buf = getattr(L, name)
            if buf is not None:
                buf.view(torch.uint8).fill_(0x5A)
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(L)
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"replay {rep}: {k} differs"
        step()
        torch.cuda.synchronize()
        got = _outputs(L)
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"eager after replay {rep}: {k} differs"
        log(f"graph replay {rep} ({activation}, fused={fused}, noalloc={noalloc}) identical "
            f"to the eager step")


@pytest.mark.parametrize("activation,fused,noalloc", CASES)
def test_layer_step_second_stream_matches_one_stream(activation, fused, noalloc):
    """The step with its backward's second stream (the router-weight gradient and the folds
    beside the DGRAD GEMMs, joined by events; on by default only for large steps, forced on
    here) gives every output bit for bit as the step in one stream, over several steps in a
    row."""
    from balanced_token_dispatch_amd.layer import LayerStep, Shape
    d = synth.Dims(R=8, S=512, K=4, E=32, B=4, H=256, Hp=192)
    idx, w = synth.routing(d, 1.0, 22)
    L = LayerStep(Shape(d.R, d.S, d.K, d.E, d.B, d.H, d.Hp), rank=2, activation=activation,
                  fused_gather=fused, plan_noalloc=noalloc, overlap=True)
    for t, sd in ((L.x_all, 221), (L.y_all, 224), (L.dout_all, 225), (L.dxp_all, 226)):
        synth.fill_normal_(t, 1.0, sd)
    synth.fill_normal_(L.w_up, 0.05, 222)
    synth.fill_normal_(L.w_down, 0.05, 223)
    L.topk_idx.copy_(torch.from_numpy(idx))
    L.topk_w.copy_(torch.from_numpy(w))

    def step(overlap):
        L.overlap = overlap
        L.dw_up.zero_()
        L.dw_down.zero_()
        L.step()
        torch.cuda.synchronize()
        return _outputs(L)

    ref = step(False)
    assert int(L.status.item()) == 0
    for rep in range(3):
        got = step(True)
        for k, v in ref.items():
            same = torch.equal(got[k].view(torch.uint8), v.view(torch.uint8))
            log(f"second stream {activation} fused={fused} rep={rep} {k}: "
                f"{'identical' if same else 'DIFFERENT'}")
            assert same, k
