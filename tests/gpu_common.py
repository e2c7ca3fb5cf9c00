"""Helpers shared by the GPU parity tests: device buffers, the HIP path through the C ABI,
tolerance checks.  Inputs come from synth; expected values from the oracle only."""
import sys

import numpy as np
import torch

import oracle

POISON = 0x7F7F7F7F


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def mod():
    import balanced_token_dispatch_amd as m
    return m


def bits(t):
    """bf16 tensor -> uint16 numpy bits (host); fp32 -> float32 numpy."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def from_bits(a, device="cuda"):
    """uint16 bf16 bits or float32 numpy -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def poisoned(shape, dtype, device="cuda"):
    t = torch.empty(shape, dtype=dtype, device=device)
    t.view(torch.uint8).fill_(0x7F)
    return t


class GpuPlan:
    """Run moe_plan + moe_dispatch_layout for one rank through the C ABI."""

    def __init__(self, R, S, K, E, B):
        m = mod()
        self.m = m
        self.d = m.dims(R, S, K, E, B)
        self.R, self.S, self.K, self.E, self.B = R, S, K, E, B
        self.SK = S * K
        self.G = E + B
        self.counts = poisoned((R, E), torch.int32)
        self.plan = poisoned((m.plan_words(self.d),), torch.int32)
        self.status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        self.ws_plan = torch.empty(m.plan_workspace_bytes(self.d), dtype=torch.uint8, device="cuda")
        self.ws_lay = torch.empty(m.dispatch_layout_workspace_bytes(self.d), dtype=torch.uint8,
                                  device="cuda")
        self.cu = poisoned((self.G + 1,), torch.int32)
        self.dest = poisoned((R * self.SK,), torch.int32)
        self.src = poisoned((self.SK,), torch.int32)

    def run(self, topk_dev, rank):
        self.m.moe_plan(self.d, topk_dev, self.counts, self.plan, self.status, self.ws_plan)
        self.m.moe_dispatch_layout(self.d, rank, topk_dev, self.plan, self.cu, self.dest, self.src,
                                   self.ws_lay)

    def host(self):
        torch.cuda.synchronize()
        return (self.counts.cpu().numpy(), self.plan.cpu().numpy(), int(self.status.item()),
                self.cu.cpu().numpy(), self.dest.cpu().numpy(), self.src.cpu().numpy())


def check_plan_layout(gp, topk_np, rank, pl=None):
    """Bit-exact comparison of plan blob, counts, cu_seqlens, dest_pos, src_flat vs the oracle."""
    if pl is None:
        pl = oracle.plan(topk_np, gp.E, gp.B)
    counts, blob, status, cu, dest, src = gp.host()
    ref_blob = pl.to_blob()
    assert (counts == pl.counts).all(), "counts"
    if not (blob == ref_blob).all():
        bad = np.nonzero(blob != ref_blob)[0]
        raise AssertionError(f"plan blob differs at words {bad[:20]}: got {blob[bad[:20]]} "
                             f"want {ref_blob[bad[:20]]}")
    assert status == pl.status
    rcu, rdest, rsrc = oracle.layout(topk_np, pl, rank)
    assert (cu == rcu).all(), f"cu_seqlens {cu} vs {rcu}"
    if not (dest == rdest).all():
        bad = np.nonzero(dest != rdest)[0]
        raise AssertionError(f"dest_pos differs at {bad[:10]}: {dest[bad[:10]]} vs {rdest[bad[:10]]}")
    assert (src == rsrc).all(), "src_flat"
    return pl


def rel_inf(got, ref):
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    den = np.abs(r).max()
    return float(np.abs(g - r).max() / (den if den > 0 else 1.0))


def check_close(got_bits, ref_bits, dtype, tol=None, min_identical=0.98, what=""):
    """Normwise max relative error ||y - y_ref||_inf / ||y_ref||_inf within tol.

    bf16: tol 2e-2 and at least ``min_identical`` of the elements bit-identical (an fp32
    accumulation differs from the oracle's float64 sum only in rare last-place roundings);
    fp32: tol 1e-5.
    """
    if dtype == "bf16":
        tol = 2e-2 if tol is None else tol
        got = oracle.bf16_bits_to_f64(got_bits)
        ref = oracle.bf16_bits_to_f64(ref_bits)
        same = float((np.asarray(got_bits) == np.asarray(ref_bits)).mean()) if got.size else 1.0
        assert same >= min_identical, f"{what}: only {same:.4f} of elements identical"
    else:
        tol = 1e-5 if tol is None else tol
        got, ref = np.asarray(got_bits, np.float64), np.asarray(ref_bits, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = rel_inf(got, ref)
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"
    return err


def router_grad_bound(y, dest, dout, rank, S, K, dtype, width, tokens=None):
    """Error bound of the GPU router-weight gradient against the float64 definition.

    Each GPU thread sums its 16-byte vectors of the row in order (ceil(vec/256) vectors of
    8 bf16 or 4 fp32 products), then 6 butterfly levels and the 4 waves of the block add up
    the partial sums: n = terms per thread + 8 fp32 roundings on any path, so
    |err| <= n * 2^-24 * sum_h |g_h y_h|, plus half an ulp for the reference's own rounding
    to float32.  Returns the [tokens, K] bound.
    """
    wide = (lambda a: oracle.bf16_bits_to_f64(a)) if dtype == "bf16" else (lambda a: np.asarray(a, np.float64))
    per_vec = 8 if dtype == "bf16" else 4
    vec = width // per_vec
    n = ((vec + 255) // 256) * per_vec + 8
    toks = np.arange(S) if tokens is None else np.asarray(tokens)
    bound = np.zeros((toks.size, K))
    dp = np.asarray(dest).reshape(-1)
    for t, s_ in enumerate(toks):
        gs = np.abs(wide(dout[int(s_)]))
        for k in range(K):
            dd = int(dp[(rank * S + int(s_)) * K + k])
            if dd >= 0:
                bound[t, k] = n * 2.0 ** -24 * float(np.dot(gs, np.abs(wide(y[dd]))))
    return bound + 1e-30


def within_one_bf16_ulp(got_bits, ref_bits, what=""):
    """Every element within one bf16 rounding step of the reference.

    For results computed in fp32 (relative error ~1e-6, far below bf16's half-ulp of 2^-9)
    and rounded once, the rounded values can differ only where the exact value sits next to
    a rounding boundary, and then by one unit in the last place.
    """
    g = oracle.bf16_bits_to_f64(np.asarray(got_bits))
    r = oracle.bf16_bits_to_f64(np.asarray(ref_bits))
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    mag = np.maximum(np.abs(g), np.abs(r))
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0.0)
    bad = np.abs(g - r) > ulp + 1e-30
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond one ulp, e.g. {g[bad][:4]} vs {r[bad][:4]}"
