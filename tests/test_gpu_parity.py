"""HIP path vs the CPU oracle, through the C ABI, at sizes the oracle finishes in seconds.

Plan, layout, permute, fold and prefetch must match bit for bit; GEMM and combine match
bit for bit on small-integer inputs (every fp32 partial sum exact) and within the stated
tolerance on random inputs (normwise max relative error 2e-2 in bf16, 1e-5 in fp32).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import (GpuPlan, bits, check_close, check_plan_layout, from_bits, log, mod,
                        router_grad_bound, within_one_bf16_ulp,
                        poisoned)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mod()  # fails loudly if the library is missing


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------------------------------------
# plan + dispatch layout (bit-exact)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["plan_g1_single_donor.json", "plan_g2_split_piece.json",
                                  "plan_g3_ties_overflow.json", "plan_g4_bad_id.json"])
def test_plan_layout_golden(name):
    g = json.load(open(os.path.join(GOLDEN, name)))
    idx = np.array(g["topk_idx"], np.int32)
    Bs = [c["B"] for c in g["cases"]] if "cases" in g else [g["B"]]
    for B in Bs:
        gp = GpuPlan(g["R"], g["S"], g["K"], g["E"], B)
        for r in range(g["R"]):
            log(f"golden {name} B={B} rank={r}")
            gp.run(_dev(idx), r)
            check_plan_layout(gp, idx, r)


def _random_routing(rng, R, S, K, E, skew):
    pop = rng.dirichlet(np.full(E, skew))
    out = np.empty((R, S, K), np.int32)
    for p in range(R):
        # K distinct experts per token via Gumbel top-K on log-popularity
        g = np.log(pop)[None, :] + rng.gumbel(size=(S, E))
        out[p] = np.argsort(-g, axis=1)[:, :K]
    return out


CASES = [
    # R, S, K, E, B, skew
    (1, 300, 3, 12, 2, 1.0),
    (2, 5000, 2, 8, 2, 0.5),         # several chunks + ragged tail
    (4, 128, 2, 16, 2, 0.3),
    (8, 1000, 6, 64, 4, 5.0),
    (8, 3000, 4, 64, 1, 0.2),        # likely slot overflow
    (16, 257, 8, 128, 8, 0.5),
    (32, 512, 8, 256, 8, 1.0),
    (64, 130, 8, 384, 8, 0.3),
    (5, 999, 3, 20, 0, 0.5),         # B = 0
    (512, 16, 2, 1024, 4, 0.5),      # maximum R and E
    (4, 1, 1, 4, 1, 0.5),            # one token per rank, K = 1, one expert per rank
    (6, 33, 1, 6, 3, 5.0),           # K = 1, one expert per rank, near-uniform routing
    (3, 40, 6, 6, 2, 0.5),           # K = E: every token on every expert, exactly balanced
    (2, 2049, 2, 4, 1, 0.4),         # S*K = 4098: two full layout chunks and a 2-copy tail
]


@pytest.mark.parametrize("case", CASES)
def test_plan_layout_random(case):
    R, S, K, E, B, skew = case
    rng = np.random.default_rng(R * 1000 + S)
    idx = _random_routing(rng, R, S, K, E, skew)
    gp = GpuPlan(R, S, K, E, B)
    pl = oracle.plan(idx, E, B)
    for r in sorted({0, R // 2, R - 1}):
        log(f"random plan case={case} rank={r} status={pl.status} replicas={len(pl.replicas)}")
        gp.run(_dev(idx), r)
        check_plan_layout(gp, idx, r, pl)


RELAY_CASES = [
    # R, S, K, E, B, skew: routings whose walk needs more than B slots on some rank
    (4, 64, 2, 8, 1, 0.3),           # one relay
    (8, 200, 2, 16, 1, 0.3),
    (8, 50, 1, 8, 1, 0.5),
    (16, 100, 4, 32, 1, 0.2),        # relays drop replicas; the bounded search plans it
    (32, 256, 8, 256, 1, 0.1),       # the same at 32 ranks
    (64, 64, 4, 128, 1, 0.1),        # 13 relays over 64 ranks
]


@pytest.mark.parametrize("case", RELAY_CASES)
def test_plan_layout_relay(case):
    """The relay fallback (walk replicas re-placed through donors) matches the oracle bit for
    bit: plan blob, cu_seqlens, dest_pos and src_flat."""
    R, S, K, E, B, skew = case
    rng = np.random.default_rng(R * 1000 + S)
    with np.errstate(divide="ignore"):
        idx = _random_routing(rng, R, S, K, E, skew)
    pl = oracle.plan(idx, E, B)
    assert pl.max_needed > B and pl.n_relayed > 0
    gp = GpuPlan(R, S, K, E, B)
    for r in sorted({0, 1, R // 2, R - 1}):
        log(f"relay plan case={case} rank={r} status={pl.status} relayed={pl.n_relayed}")
        gp.run(_dev(idx), r)
        check_plan_layout(gp, idx, r, pl)


def test_plan_layout_relay_seeded_overflows():
    """Every walk overflow of the oracle's seeded medium-routing set (4-8 ranks, 1-4 experts
    per rank, B = 1..3; the set the CPU test pins against mixed-integer feasibility), solved or
    not, and of 300 more routings of 6-16 ranks: the GPU plan and layout match the oracle bit for
    bit (first and last rank of the first set, rank 0 of the second), among them the plans the
    bounded search finds where the relay fallback drops a replica."""
    from test_oracle_plan import random_routing
    n = searched = 0
    for seed in range(60):
        rng = np.random.default_rng(10_000 + seed)
        R = int(rng.integers(4, 9))
        E_loc = int(rng.choice([1, 2, 4]))
        E = R * E_loc
        K = int(rng.integers(1, min(E, 4) + 1))
        S = int(rng.integers(2, 32))
        idx = random_routing(rng, R, S, K, E, skew=float(rng.choice([0.5, 1.0, 2.0, 5.0])))
        for B in (1, 2, 3):
            pl = oracle.plan(idx, E, B)
            if pl.max_needed <= B:
                continue
            n += 1
            searched += pl.n_search > 0 and pl.status == 0
            gp = GpuPlan(R, S, K, E, B)
            for r in (0, R - 1):
                gp.run(_dev(idx), r)
                check_plan_layout(gp, idx, r, pl)
    # and 300 routings of 6-16 ranks with stronger skew
    for seed in range(300):
        rng = np.random.default_rng(50_000 + seed)
        R = int(rng.integers(6, 17))
        E_loc = int(rng.choice([1, 2, 4]))
        E = R * E_loc
        K = int(rng.integers(1, min(E, 6) + 1))
        S = int(rng.integers(2, 40))
        idx = random_routing(rng, R, S, K, E, skew=float(rng.choice([1.0, 2.0, 5.0, 10.0])))
        for B in (1, 2):
            pl = oracle.plan(idx, E, B)
            if pl.max_needed <= B:
                continue
            n += 1
            searched += pl.n_search > 0 and pl.status == 0
            gp = GpuPlan(R, S, K, E, B)
            gp.run(_dev(idx), 0)
            check_plan_layout(gp, idx, 0, pl)
    log(f"relay: {n} seeded overflows bit-exact, {searched} of them planned by the search")
    assert n >= 400 and searched >= 20


@pytest.mark.parametrize("seed", [0, 11, 13])
def test_plan_layout_search_gives_up(seed):
    """32-64 ranks, B = 1, skew up to 20: routings where the relay fallback drops replicas and
    the bounded search finds no plan, at once (seeds 0, 13: some receiver's deficit exceeds
    every expert it could take from) or after its 4096 placements (seed 11).  The relay
    fallback's plan stands, with MOE_DEV_SLOT_OVERFLOW, bit for bit as in the oracle."""
    from test_oracle_plan import random_routing
    rng = np.random.default_rng(90_000 + seed)
    R = int(rng.choice([32, 64]))
    E_loc = int(rng.choice([2, 4, 8]))
    E = R * E_loc
    K = int(rng.choice([4, 8]))
    S = int(rng.integers(16, 128))
    idx = random_routing(rng, R, S, K, E, skew=float(rng.choice([2.0, 5.0, 10.0, 20.0])))
    pl = oracle.plan(idx, E, 1)
    assert pl.status & oracle.STATUS_SLOT_OVERFLOW
    assert pl.n_search == (oracle.moe_ref.SEARCH_BUDGET if seed == 11 else 0)
    gp = GpuPlan(R, S, K, E, 1)
    for r in (0, R - 1):
        log(f"search gives up seed={seed} R={R} E={E} rank={r} steps={pl.n_search}")
        gp.run(_dev(idx), r)
        check_plan_layout(gp, idx, r, pl)


def test_plan_layout_search_gives_up_max_shape():
    """R = 512, E = 1024 (the largest the library takes), B = 1, skew 20: the search spends its
    whole budget and the relay fallback's plan stands, bit for bit as in the oracle."""
    from test_oracle_plan import random_routing
    rng = np.random.default_rng(77_000)
    R, E, K = 512, 1024, 4
    S = int(rng.integers(8, 32))
    idx = random_routing(rng, R, S, K, E, skew=float(rng.choice([5.0, 10.0, 20.0])))
    pl = oracle.plan(idx, E, 1)
    assert pl.status & oracle.STATUS_SLOT_OVERFLOW and pl.n_search == oracle.moe_ref.SEARCH_BUDGET
    gp = GpuPlan(R, S, K, E, 1)
    for r in (0, R - 1):
        log(f"search gives up at R={R} E={E} rank={r}")
        gp.run(_dev(idx), r)
        check_plan_layout(gp, idx, r, pl)


@pytest.mark.parametrize("B", [1, 2])
def test_plan_layout_relay_chain(B):
    """Five donors with excess 1 and one receiver with deficit 5: chains of relays (B=2) and
    of switches (B=1) re-place every piece; all ranks checked."""
    R, K, S, E = 6, 1, 5, 6
    flat = []
    for r in range(1, R):
        flat += [r] * (S + 1)
    idx = np.array(flat, np.int32).reshape(R, S, K)
    pl = oracle.plan(idx, E, B)
    assert pl.status == 0 and pl.n_relayed > 0
    gp = GpuPlan(R, S, K, E, B)
    for r in range(R):
        gp.run(_dev(idx), r)
        check_plan_layout(gp, idx, r, pl)


def test_plan_layout_bad_ids():
    rng = np.random.default_rng(11)
    R, S, K, E, B = 4, 700, 3, 16, 3
    idx = _random_routing(rng, R, S, K, E, 0.5)
    idx[0, 5, 1] = -7
    idx[3, 699, 2] = E
    idx[2, 100, 0] = 1 << 30
    gp = GpuPlan(R, S, K, E, B)
    for r in range(R):
        gp.run(_dev(idx), r)
        pl = check_plan_layout(gp, idx, r)
        assert pl.status & oracle.STATUS_BAD_EXPERT_ID


@pytest.mark.parametrize("wl", ["tiny_f32", "balanced_bf16"])
def test_plan_layout_workloads(wl):
    w = synth.WORKLOADS[wl]
    d = w.dims
    idx, _ = synth.routing(d, synth.zipf_for(w, w.maxvio_targets[0]), w.base_seed)
    gp = GpuPlan(d.R, d.S, d.K, d.E, d.B)
    pl = oracle.plan(idx, d.E, d.B)
    assert pl.status == 0
    for r in range(d.R):
        gp.run(_dev(idx), r)
        check_plan_layout(gp, idx, r, pl)


def test_plan_layout_exactly_balanced():
    d = synth.WORKLOADS["balanced_bf16"].dims
    idx, _ = synth.balanced_routing(d)
    gp = GpuPlan(d.R, d.S, d.K, d.E, d.B)
    gp.run(_dev(idx), 0)
    pl = check_plan_layout(gp, idx, 0)
    assert pl.replicas == []


# ------------------------------------------------------------------------------------------
# permute, combine, fold, prefetch
# ------------------------------------------------------------------------------------------

def _plan_for(R, S, K, E, B, seed, skew=0.5):
    rng = np.random.default_rng(seed)
    idx = _random_routing(rng, R, S, K, E, skew)
    return idx, oracle.plan(idx, E, B)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scaled", [False, True])
@pytest.mark.parametrize("S", [300, 301])   # S*K even and odd (the weighted form pairs rows)
def test_permute(dtype, scaled, S):
    R, K, E, B, H = 4, 3, 16, 1, 136
    idx, pl = _plan_for(R, S, K, E, B, 3, skew=0.2)
    m = mod()
    d = m.dims(R, S, K, E, B)
    rank = 0
    _, _, src = oracle.layout(idx, pl, rank)
    x = synth.host_normal(7, 1, (R * S, H))
    x = synth.to_bf16_bits(x) if dtype == "bf16" else x
    w = synth.routing(synth.Dims(R, S, K, E, B, H, H), 0.3, 9)[1].reshape(-1)
    xd = from_bits(x)
    xp = poisoned((S * K, H), xd.dtype)
    m.moe_permute(d, xd, _dev(src), xp, row_scale=_dev(w) if scaled else None)
    ref = oracle.permute(x, src, K, row_scale=w if scaled else None, dtype=dtype)
    got = bits(xp)
    assert (got.view(np.uint8) == ref.view(np.uint8)).all()
    if pl.status:
        assert (src == -1).any() and (got[src == -1] == 0).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K", [2, 8, 17])
def test_combine(dtype, K):
    R, S, E, B, W = 3, 200, 24, 2, 264
    idx, pl = _plan_for(R, S, K, E, B, 5 + K)
    m = mod()
    d = m.dims(R, S, K, E, B)
    _, dest, _ = oracle.layout(idx, pl, 0)
    dest = dest.copy()
    dest[::37] = -1                          # copies without a destination add nothing
    w = np.random.default_rng(1).random(R * S * K).astype(np.float32)
    y = synth.host_normal(8, 2, (R * S * K, W))
    y = synth.to_bf16_bits(y) if dtype == "bf16" else y
    for rank in (0, R - 1):
        out = poisoned((S, W), torch.bfloat16 if dtype == "bf16" else torch.float32)
        m.moe_combine(d, rank, from_bits(y), _dev(dest), _dev(w), out)
        ref = oracle.combine(y, dest, w, rank, S, K, dtype)
        check_close(bits(out), ref, dtype, what=f"combine K={K} rank={rank}")


def test_combine_integer_exact():
    R, S, K, E, B, W = 4, 128, 8, 32, 4, 512
    idx, pl = _plan_for(R, S, K, E, B, 21)
    m = mod()
    d = m.dims(R, S, K, E, B)
    _, dest, _ = oracle.layout(idx, pl, 1)
    w = np.random.default_rng(2).choice(np.array([0.25, 0.5, 1.0], np.float32), R * S * K)
    y = synth.to_bf16_bits(synth.host_ternary(3, 3, (R * S * K, W)))
    out = poisoned((S, W), torch.bfloat16)
    m.moe_combine(d, 1, from_bits(y), _dev(dest), _dev(w), out)
    assert (bits(out) == oracle.combine(y, dest, w, 1, S, K, "bf16")).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K", [2, 8, 17])
def test_unpermute_reduce(dtype, K):
    R, S, E, B, W = 3, 200, 24, 2, 264
    idx, pl = _plan_for(R, S, K, E, B, 7 + K)
    m = mod()
    d = m.dims(R, S, K, E, B)
    _, dest, _ = oracle.layout(idx, pl, 0)
    dest = dest.copy()
    dest[5::41] = -1                         # copies without a destination add nothing
    g = synth.host_normal(12, 2, (R * S * K, W))
    g = synth.to_bf16_bits(g) if dtype == "bf16" else g
    for rank in (0, R - 1):
        dx = poisoned((S, W), torch.bfloat16 if dtype == "bf16" else torch.float32)
        m.moe_unpermute_reduce(d, rank, from_bits(g), _dev(dest), dx)
        ref = oracle.unpermute_reduce(g, dest, rank, S, K, dtype)
        check_close(bits(dx), ref, dtype, what=f"unpermute reduce K={K} rank={rank}")


@pytest.mark.parametrize("dtype,W", [("bf16", 16400), ("f32", 8216)])
def test_combine_and_unpermute_wide_rows(dtype, W):
    """Rows wider than one block takes (2050 and 2054 vectors of 16 bytes: a second block per
    row covers the last few vectors), K = 3, both weighted and unweighted forms."""
    R, S, K, E, B = 2, 24, 3, 8, 1
    idx, pl = _plan_for(R, S, K, E, B, 31)
    m = mod()
    d = m.dims(R, S, K, E, B)
    _, dest, _ = oracle.layout(idx, pl, 0)
    dest = dest.copy()
    dest[4::13] = -1
    w = np.random.default_rng(2).random(R * S * K).astype(np.float32)
    y = synth.host_normal(13, 2, (R * S * K, W))
    y = synth.to_bf16_bits(y) if dtype == "bf16" else y
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for rank in (0, R - 1):
        out = poisoned((S, W), tdt)
        m.moe_combine(d, rank, from_bits(y), _dev(dest), _dev(w), out)
        check_close(bits(out), oracle.combine(y, dest, w, rank, S, K, dtype), dtype,
                    what=f"wide combine rank={rank}")
        dx = poisoned((S, W), tdt)
        m.moe_unpermute_reduce(d, rank, from_bits(y), _dev(dest), dx)
        check_close(bits(dx), oracle.unpermute_reduce(y, dest, rank, S, K, dtype), dtype,
                    what=f"wide unpermute reduce rank={rank}")


def test_unpermute_reduce_integer_exact():
    R, S, K, E, B, W = 4, 128, 8, 32, 4, 520
    idx, pl = _plan_for(R, S, K, E, B, 22)
    m = mod()
    d = m.dims(R, S, K, E, B)
    _, dest, _ = oracle.layout(idx, pl, 2)
    g = synth.to_bf16_bits(synth.host_ternary(4, 3, (R * S * K, W)))
    dx = poisoned((S, W), torch.bfloat16)
    m.moe_unpermute_reduce(d, 2, from_bits(g), _dev(dest), dx)
    assert (bits(dx) == oracle.unpermute_reduce(g, dest, 2, S, K, "bf16")).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K,W", [(2, 264), (8, 1064), (17, 4104)])
def test_combine_weight_grad(dtype, K, W):
    R, S, E, B = 3, 150, 24, 2
    idx, pl = _plan_for(R, S, K, E, B, 13 + K)
    m = mod()
    d = m.dims(R, S, K, E, B)
    _, dest, _ = oracle.layout(idx, pl, 0)
    dest = dest.copy()
    dest[3::29] = -1
    y = synth.host_normal(14, 2, (R * S * K, W))
    gout = synth.host_normal(15, 3, (S, W))
    if dtype == "bf16":
        y, gout = synth.to_bf16_bits(y), synth.to_bf16_bits(gout)
    for rank in (0, R - 1):
        dw = poisoned((S * K,), torch.float32)
        m.moe_combine_weight_grad(d, rank, from_bits(y), _dev(dest), from_bits(gout), dw)
        got = dw.cpu().numpy().reshape(S, K)
        ref = oracle.combine_weight_grad(y, dest, gout, rank, S, K, dtype)
        none = np.asarray(dest).reshape(R, S, K)[rank] < 0
        assert (got[none] == 0).all(), "copies without a destination get a zero gradient"
        bound = router_grad_bound(y, dest, gout, rank, S, K, dtype, W)
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        # the oracle's float32 rounding of its float64 result adds half an ulp
        assert (err <= bound + np.abs(ref) * 2.0 ** -24).all(), f"max excess {(err - bound).max()}"


def test_combine_weight_grad_integer_exact():
    R, S, K, E, B, W = 4, 96, 8, 32, 4, 2048
    idx, pl = _plan_for(R, S, K, E, B, 23)
    m = mod()
    d = m.dims(R, S, K, E, B)
    _, dest, _ = oracle.layout(idx, pl, 3)
    y = synth.to_bf16_bits(synth.host_ternary(5, 3, (R * S * K, W)))
    gout = synth.to_bf16_bits(synth.host_ternary(6, 4, (S, W)))
    dw = poisoned((S * K,), torch.float32)
    m.moe_combine_weight_grad(d, 3, from_bits(y), _dev(dest), from_bits(gout), dw)
    ref = oracle.combine_weight_grad(y, dest, gout, 3, S, K, "bf16")
    assert (dw.cpu().numpy().reshape(S, K) == ref).all()


def test_fold_and_prefetch():
    R, S, K, E, B = 8, 400, 4, 32, 4
    idx, pl = _plan_for(R, S, K, E, B, 31, skew=0.3)
    m = mod()
    d = m.dims(R, S, K, E, B)
    plan_d = _dev(pl.to_blob())
    row = 8 * 24
    for rank in range(R):
        dw = synth.host_normal(rank, 4, (E + B, row))
        dwd = _dev(dw)
        m.moe_replica_grad_fold(d, rank, plan_d, dwd)
        assert (dwd.cpu().numpy() == oracle.replica_grad_fold(dw, pl, rank)).all()
        wt = synth.to_bf16_bits(synth.host_normal(rank, 5, (E + B, 8, 24)))
        wd = from_bits(wt)
        m.moe_prefetch(d, rank, plan_d, wd)
        assert (bits(wd) == oracle.prefetch(wt, pl, rank)).all()
    assert any(m_.slot >= 0 for m_ in pl.replicas)


# ------------------------------------------------------------------------------------------
# grouped GEMM
# ------------------------------------------------------------------------------------------

def _segments(rng, G, M_total, empties=True):
    cuts = np.sort(rng.integers(0, M_total + 1, size=G - 1))
    cu = np.concatenate([[0], cuts, [M_total]]).astype(np.int32)
    if empties and G > 3:
        cu[2] = cu[1]  # an empty segment
    return cu


def _gemm_inputs(op, G, M, Kd, N, dtype, gen):
    """a, b for the op; gen(tag, shape) -> float32 array."""
    if op == "fwd":
        a, b = gen(1, (M, Kd)), gen(2, (G, Kd, N))
    elif op == "dgrad":
        a, b = gen(1, (M, N)), gen(2, (G, Kd, N))
    else:
        a, b = gen(1, (M, Kd)), gen(2, (M, N))
    if dtype == "bf16":
        a, b = synth.to_bf16_bits(a), synth.to_bf16_bits(b)
    return a, b


def _gemm_ws(m, op):
    """A GEMM workspace filled with 0xFF bytes (NaN floats), to see whether it was written."""
    n = m.group_gemm_workspace_bytes(op)
    return torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")


def _run_gemm(op, a, b, cu, Kd, N, dtype, out_init=None, ws=None):
    m = mod()
    opc = {"fwd": m.GEMM_FWD, "dgrad": m.GEMM_DGRAD, "wgrad": m.GEMM_WGRAD}[op]
    ad, bd, cud = from_bits(a), from_bits(b), _dev(cu)
    M = a.shape[0]
    G = cu.size - 1
    if op == "wgrad":
        out = _dev(out_init.astype(np.float32))
    else:
        cols = N if op == "fwd" else Kd
        out = poisoned((M, cols), torch.bfloat16 if dtype == "bf16" else torch.float32)
    m.moe_group_gemm(opc, ad, bd, cud, out, Kd, N, ws)
    return bits(out) if op != "wgrad" else out.cpu().numpy()


GEMM_SHAPES = [
    # G, M, Kd, N
    (5, 700, 64, 256),
    (6, 1000, 136, 392),      # Kd, N not multiples of the tile
    (18, 600, 256, 512),
    (3, 2100, 520, 264),
    (9, 257, 1408, 2048),
    (1, 300, 96, 96),         # one segment, one partial tile
    (1088, 3000, 64, 128),    # the largest G: ~3 rows per segment, many empty
    (2, 500, 32, 320),        # a one-step contraction
]


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_group_gemm_integer_exact(op, shape):
    G, M, Kd, N = shape
    rng = np.random.default_rng(G * 7 + M)
    cu = _segments(rng, G, M - 3)           # a few rows outside every segment
    a, b = _gemm_inputs(op, G, M, Kd, N, "bf16",
                        lambda t, s: synth.host_ternary(G + M, t, s))
    init = synth.host_ternary(G, 9, (G, Kd, N)) if op == "wgrad" else None
    log(f"gemm int op={op} shape={shape}")
    got = _run_gemm(op, a, b, cu, Kd, N, "bf16", init)
    ref = oracle.group_gemm(op, a, b, cu, "bf16", out=init)
    if op == "wgrad":
        assert (got == ref).all()
    else:
        rows = cu[-1]
        assert (got[:rows] == ref[:rows]).all()
        assert (got[rows:].view(np.uint16) == 0x7F7F).all(), "rows outside segments untouched"


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
@pytest.mark.parametrize("shape", GEMM_SHAPES[:4])
def test_group_gemm_random_bf16(op, shape):
    G, M, Kd, N = shape
    rng = np.random.default_rng(G * 11 + M)
    cu = _segments(rng, G, M)
    a, b = _gemm_inputs(op, G, M, Kd, N, "bf16",
                        lambda t, s: synth.host_normal(G + M, t, s, 1.0 if t == 1 else 0.05))
    init = synth.host_normal(G, 9, (G, Kd, N)) if op == "wgrad" else None
    got = _run_gemm(op, a, b, cu, Kd, N, "bf16", init)
    ref = oracle.group_gemm(op, a, b, cu, "bf16", out=init)
    if op == "wgrad":
        err = float(np.abs(got - ref).max() / np.abs(ref).max())
        assert err <= 1e-4, err
    else:
        check_close(got, ref, "bf16", what=f"gemm {op} {shape}")


# Shapes whose last round of tiles the kernel splits over the workgroups when given a
# workspace (64 or more K steps per tile, leftover tiles well under a round of 256 CUs).
SPLIT_CASES = [
    # op, G, M, Kd, N
    ("fwd", 5, 3000, 2048, 256),      # ~14 tiles, no whole round: every tile split
    ("fwd", 4, 1500, 2056, 512),      # ragged contraction: 65 K steps, the last one partial
    ("dgrad", 3, 2100, 256, 2048),
    ("dgrad", 6, 1800, 520, 2056),    # ragged contraction, a partial column tile
    ("fwd", 3, 66000, 2048, 256),     # more tiles than a round: whole rounds, then the split
]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_group_gemm_split_round_integer_exact(case):
    """Ternary inputs: every partial sum is exact, so the split result is the oracle's, bit for
    bit, and equal to the unsplit kernel's; the workspace was used."""
    op, G, M, Kd, N = case
    m = mod()
    rng = np.random.default_rng(G * 13 + M)
    cu = _segments(rng, G, M - 3)
    a, b = _gemm_inputs(op, G, M, Kd, N, "bf16", lambda t, s: synth.host_ternary(G + M, t, s))
    ws = _gemm_ws(m, m.GEMM_FWD if op == "fwd" else m.GEMM_DGRAD)
    log(f"gemm split op={op} shape={case[1:]}")
    got = _run_gemm(op, a, b, cu, Kd, N, "bf16", ws=ws)
    assert (ws != 0xFF).any(), "the last round was not split"
    plain = _run_gemm(op, a, b, cu, Kd, N, "bf16")
    ref = oracle.group_gemm(op, a, b, cu, "bf16")
    rows = cu[-1]
    assert (got[:rows] == ref[:rows]).all()
    assert (got == plain).all()
    assert (got[rows:].view(np.uint16) == 0x7F7F).all(), "rows outside segments untouched"


@pytest.mark.parametrize("case", SPLIT_CASES[:4])
def test_group_gemm_split_round_random(case):
    """Random inputs: within the bf16 tolerance of the oracle, close to the unsplit result,
    and the same on a second call."""
    op, G, M, Kd, N = case
    m = mod()
    rng = np.random.default_rng(G * 17 + M)
    cu = _segments(rng, G, M)
    a, b = _gemm_inputs(op, G, M, Kd, N, "bf16",
                        lambda t, s: synth.host_normal(G + M, t, s, 1.0 if t == 1 else 0.05))
    ws = _gemm_ws(m, m.GEMM_FWD if op == "fwd" else m.GEMM_DGRAD)
    got = _run_gemm(op, a, b, cu, Kd, N, "bf16", ws=ws)
    again = _run_gemm(op, a, b, cu, Kd, N, "bf16", ws=ws)
    assert (got == again).all()
    ref = oracle.group_gemm(op, a, b, cu, "bf16")
    check_close(got, ref, "bf16", what=f"split gemm {op} {case[1:]}")
    # the split changes only the fp32 summation order of the last round's tiles: the two
    # results differ in rare last-place roundings
    plain = _run_gemm(op, a, b, cu, Kd, N, "bf16")
    check_close(got[:cu[-1]], plain[:cu[-1]], "bf16", tol=1e-2, min_identical=0.98,
                what="split vs unsplit")


def test_group_gemm_swiglu_split_round():
    """The gated FWD with a split last round: pre-activation exact on ternary inputs, z within
    one bf16 unit of the oracle, both equal to the unsplit call's."""
    rng = np.random.default_rng(5)
    G, M, Kd, N = 4, 2500, 2048, 512
    m = mod()
    cu = _segments(rng, G, M)
    a = synth.to_bf16_bits(synth.host_ternary(2, 1, (M, Kd)))
    W = synth.to_bf16_bits(synth.host_ternary(2, 2, (G, Kd, N)))
    ws = _gemm_ws(m, m.GEMM_FWD)
    z, h = poisoned((M, N // 2), torch.bfloat16), poisoned((M, N), torch.bfloat16)
    m.moe_group_gemm_swiglu(from_bits(a), from_bits(W), _dev(cu), z, h, Kd, N, ws)
    assert (ws != 0xFF).any(), "the last round was not split"
    z0, h0 = poisoned((M, N // 2), torch.bfloat16), poisoned((M, N), torch.bfloat16)
    m.moe_group_gemm_swiglu(from_bits(a), from_bits(W), _dev(cu), z0, h0, Kd, N)
    z_ref, h_ref = oracle.group_gemm_swiglu(a, W, cu, "bf16")
    rows = np.arange(cu[0], cu[-1])
    assert (bits(h)[rows] == h_ref[rows]).all()
    assert (bits(h) == bits(h0)).all() and (bits(z) == bits(z0)).all()
    within_one_bf16_ulp(bits(z)[rows], z_ref[rows], what="split swiglu z on ternary inputs")


def test_group_gemm_wgrad_unequal_segments():
    """WGRAD tiles are dealt longest segment first, rounds alternating direction: segments of
    many different lengths (repeated lengths, empty segments, one long one), about 2.6 rounds
    of tiles on 256 CUs, ternary inputs, bit for bit against the oracle."""
    G, Kd, N = 60, 768, 1024
    rng = np.random.default_rng(60)
    lens = rng.integers(1, 90, size=G)
    lens[[3, 17, 40]] = 0                    # empty segments
    lens[[5, 6, 30]] = 57                    # equal lengths
    lens[10] = 700                           # one long segment
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    M = int(cu[-1]) + 5                      # a few rows outside every segment
    a, b = _gemm_inputs("wgrad", G, M, Kd, N, "bf16",
                        lambda t, s: synth.host_ternary(61, t, s))
    init = synth.host_ternary(62, 9, (G, Kd, N))
    log(f"gemm wgrad unequal segments G={G} M={M}")
    got = _run_gemm("wgrad", a, b, cu, Kd, N, "bf16", init)
    ref = oracle.group_gemm("wgrad", a, b, cu, "bf16", out=init)
    assert (got == ref).all()


@pytest.mark.parametrize("Kd,N", [(1408, 2048), (264, 520), (1408, 136)])
def test_group_gemm_wgrad_row_edge_guard(Kd, N):
    """WGRAD tiles cut by the output's row edge (Kd % 256 != 0) write nothing outside their own
    weight row.  Between two active segments lies an empty one, whose weight row no tile owns,
    and after the last (active) weight row lies a guard region; both hold -0.0, which any
    read-add-write of a masked row (its accumulators are +0) would turn into +0.0, and must keep
    their bits.  The active rows match the oracle bit for bit (ternary inputs)."""
    m = mod()
    G = 4
    cu = np.concatenate([[0], np.cumsum([300, 0, 200, 150])]).astype(np.int32)
    M = int(cu[-1])
    a, b = _gemm_inputs("wgrad", G, M, Kd, N, "bf16",
                        lambda t, s: synth.host_ternary(Kd + N, t, s))
    init = synth.host_ternary(Kd, 9, (G, Kd, N))
    init[1] = -0.0
    n_out, n_guard = G * Kd * N, 256 * N
    full = torch.empty(n_out + n_guard, dtype=torch.float32, device="cuda")
    full.view(torch.int32).fill_(-2 ** 31)          # every word -0.0
    full[:n_out] = _dev(init.reshape(-1))
    log(f"gemm wgrad row edge Kd={Kd} N={N}")
    m.moe_group_gemm(m.GEMM_WGRAD, from_bits(a), from_bits(b), _dev(cu),
                     full[:n_out].view(G, Kd, N), Kd, N)
    got = full.cpu().numpy().view(np.uint32)
    ref = oracle.group_gemm("wgrad", a, b, cu, "bf16", out=init)
    assert (got[:n_out] == ref.reshape(-1).view(np.uint32)).all()
    assert (got[Kd * N:2 * Kd * N] == 0x80000000).all(), "empty segment's weight row untouched"
    assert (got[n_out:] == 0x80000000).all(), "guard after the last weight row untouched"


# ------------------------------------------------------------------------------------------
# fused gather GEMM: the row operand read from the token rows through the gather entries;
# the definition is the oracle's permute followed by its grouped GEMM
# ------------------------------------------------------------------------------------------

def _run_gather(op, x, gather, div, b, cu, Kd, N, out_init=None, ws=None):
    m = mod()
    opc = {"fwd": m.GEMM_FWD, "wgrad": m.GEMM_WGRAD}[op]
    if op == "wgrad":
        out = _dev(out_init.astype(np.float32))
    else:
        out = poisoned((gather.size, N), torch.bfloat16)
    xd = x if torch.is_tensor(x) else from_bits(x)
    m.moe_group_gemm_gather(opc, xd, _dev(gather), div, from_bits(b), _dev(cu), out, Kd, N, ws)
    return bits(out) if op != "wgrad" else out.cpu().numpy()


def _gather_entries(rng, cu, M, n_tok, div):
    """Copy ids of random tokens (repeats included) for the rows of every segment, -1 past
    them, as the dispatch layout writes them."""
    g = rng.integers(0, n_tok * div, size=M).astype(np.int32)
    g[cu[-1]:] = -1
    return g


GATHER_SHAPES = [
    # G, M, Kd, N, token rows, divisor
    (5, 700, 64, 256, 300, 2),
    (6, 1000, 136, 392, 97, 6),       # Kd, N not multiples of the tile; ragged contraction
    (18, 600, 256, 512, 1000, 8),
    (9, 257, 1408, 2048, 40, 17),
    (1, 300, 96, 96, 7, 1),
    (1088, 3000, 64, 128, 500, 3),    # the largest G: ~3 rows per segment, many empty
]


@pytest.mark.parametrize("op", ["fwd", "wgrad"])
@pytest.mark.parametrize("shape", GATHER_SHAPES)
def test_group_gemm_gather_integer_exact(op, shape):
    G, M, Kd, N, n_tok, div = shape
    rng = np.random.default_rng(G * 13 + M)
    cu = _segments(rng, G, M - 3)
    gather = _gather_entries(rng, cu, M, n_tok, div)
    x = synth.to_bf16_bits(synth.host_ternary(G + M, 1, (n_tok, Kd)))
    b = synth.to_bf16_bits(synth.host_ternary(G + M, 2, (G, Kd, N) if op == "fwd" else (M, N)))
    init = synth.host_ternary(G, 9, (G, Kd, N)) if op == "wgrad" else None
    log(f"gemm gather int op={op} shape={shape}")
    got = _run_gather(op, x, gather, div, b, cu, Kd, N, init)
    ref = oracle.group_gemm(op, oracle.permute(x, gather, div), b, cu, "bf16", out=init)
    if op == "wgrad":
        assert (got == ref).all()
    else:
        rows = cu[-1]
        assert (got[:rows] == ref[:rows]).all()
        assert (got[rows:].view(np.uint16) == 0x7F7F).all(), "rows outside segments untouched"


def test_group_gemm_gather_wgrad_invalid_entries():
    """WGRAD reads a gather entry that names no token row (negative, or at least
    src_rows * divisor) as a zero row, as the permute writes for a negative entry: bit-exact
    against the oracle's permute (entries past the source mapped to -1 for it) and GEMM."""
    G, M, Kd, N, n_tok, div = 7, 1500, 264, 520, 300, 4
    rng = np.random.default_rng(21)
    cu = _segments(rng, G, M - 3)
    gather = _gather_entries(rng, cu, M, n_tok, div)
    bad = rng.choice(int(cu[-1]), size=40, replace=False)
    gather[bad[:20]] = -1 - rng.integers(0, 1000, 20)
    gather[bad[20:]] = n_tok * div + rng.integers(0, 1000, 20)
    x = synth.to_bf16_bits(synth.host_ternary(3, 1, (n_tok, Kd)))
    b = synth.to_bf16_bits(synth.host_ternary(3, 2, (M, N)))
    init = synth.host_ternary(3, 9, (G, Kd, N))
    got = _run_gather("wgrad", x, gather, div, b, cu, Kd, N, init)
    g_ref = np.where((gather >= 0) & (gather < n_tok * div), gather, -1).astype(np.int32)
    ref = oracle.group_gemm("wgrad", oracle.permute(x, g_ref, div), b, cu, "bf16", out=init)
    assert (got == ref).all()


@pytest.mark.parametrize("case", [c for c in SPLIT_CASES if c[0] == "fwd"])
def test_group_gemm_gather_split_round(case):
    """The gathered FWD with a workspace splits its last round like the plain FWD: bit-exact
    on ternary inputs."""
    m = mod()
    _, G, M, Kd, N = case
    rng = np.random.default_rng(M + Kd)
    cu = _segments(rng, G, M - 2, empties=False)
    n_tok, div = M // 3 + 1, 4
    gather = _gather_entries(rng, cu, M, n_tok, div)
    x = synth.to_bf16_bits(synth.host_ternary(M, 1, (n_tok, Kd)))
    b = synth.to_bf16_bits(synth.host_ternary(M, 2, (G, Kd, N)))
    ws = _gemm_ws(m, m.GEMM_FWD)
    log(f"gemm gather split case={case}")
    got = _run_gather("fwd", x, gather, div, b, cu, Kd, N, ws=ws)
    torch.cuda.synchronize()
    assert bool((ws != 0xFF).any()), "split round not taken"
    ref = oracle.group_gemm("fwd", oracle.permute(x, gather, div), b, cu, "bf16")
    rows = cu[-1]
    assert (got[:rows] == ref[:rows]).all()


@pytest.mark.parametrize("op", ["fwd", "wgrad"])
def test_group_gemm_gather_matches_permute_then_gemm(op):
    """Random bf16 data: the gathered GEMM gives the same bits as moe_permute followed by
    moe_group_gemm (same products, same order), and is within tolerance of the oracle."""
    m = mod()
    G, M, Kd, N, n_tok, K = 12, 4000, 1024, 768, 900, 8
    rng = np.random.default_rng(77)
    cu = _segments(rng, G, M - 5)
    gather = _gather_entries(rng, cu, M, n_tok, K)
    x = synth.to_bf16_bits(synth.host_normal(5, 1, (n_tok, Kd)))
    b = synth.to_bf16_bits(synth.host_normal(5, 2, (G, Kd, N) if op == "fwd" else (M, N),
                                             0.05 if op == "fwd" else 1.0))
    init = synth.host_normal(5, 9, (G, Kd, N)) if op == "wgrad" else None
    ws = _gemm_ws(m, m.GEMM_FWD) if op == "fwd" else None
    got = _run_gather(op, x, gather, K, b, cu, Kd, N, init, ws=ws)
    # the unfused HIP path: permute into xp, then the grouped GEMM
    d = m.dims(1, M // K, K, K, 0)      # the permute's S*K rows = the M rows here
    xp = torch.empty((M, Kd), dtype=torch.bfloat16, device="cuda")
    m.moe_permute(d, from_bits(x), _dev(gather), xp)
    two = _run_gemm(op, bits(xp), b, cu, Kd, N, "bf16", init,
                    ws=_gemm_ws(m, m.GEMM_FWD) if op == "fwd" else None)
    rows = cu[-1]
    if op == "wgrad":
        assert (got.view(np.uint32) == two.view(np.uint32)).all()
    else:
        assert (got[:rows] == two[:rows]).all()
    ref = oracle.group_gemm(op, oracle.permute(x, gather, K), b, cu, "bf16", out=init)
    if op == "wgrad":
        assert float(np.abs(got - ref).max() / np.abs(ref).max()) <= 1e-4
    else:
        check_close(got[:rows], ref[:rows], "bf16", what=f"gather {op}")


@pytest.mark.parametrize("op", ["fwd", "wgrad"])
def test_group_gemm_gather_source_above_4gb(op):
    """Token rows more than 4 GB into the source buffer (past any 32-bit offset) are read
    correctly: a 4.5 GB source, gather entries drawn mostly from its last 0.5 GB."""
    G, M, Kd, N, K = 3, 600, 2048, 256, 2
    n_tok = 1_100_000                                   # 1.1e6 rows x 4 KB = 4.5 GB
    rng = np.random.default_rng(4)
    cu = np.array([0, 250, 250, 597], np.int32)
    toks = np.where(rng.random(M) < 0.8, rng.integers(1_050_000, n_tok, M),
                    rng.integers(0, n_tok, M))
    toks[0], toks[1] = n_tok - 1, 0                     # the very last and the first row
    gather = (toks * K + rng.integers(0, K, M)).astype(np.int32)
    gather[cu[-1]:] = -1
    uniq = np.unique(toks)
    rows_h = synth.to_bf16_bits(synth.host_ternary(11, 1, (uniq.size, Kd)))
    x = torch.zeros((n_tok, Kd), dtype=torch.bfloat16, device="cuda")
    x[torch.as_tensor(uniq, device="cuda")] = from_bits(rows_h)
    remap = np.full(n_tok, -1, np.int64)
    remap[uniq] = np.arange(uniq.size)
    g_local = np.where(gather >= 0, remap[np.maximum(gather, 0) // K] * K + gather % K, -1)
    b = synth.to_bf16_bits(synth.host_ternary(11, 2, (G, Kd, N) if op == "fwd" else (M, N)))
    init = np.zeros((G, Kd, N), np.float32) if op == "wgrad" else None
    log(f"gemm gather above 4 GB op={op}")
    got = _run_gather(op, x, gather, K, b, cu, Kd, N, init)
    ref = oracle.group_gemm(op, oracle.permute(rows_h, g_local.astype(np.int32), K), b, cu,
                            "bf16", out=init)
    del x
    torch.cuda.empty_cache()
    if op == "wgrad":
        assert (got == ref).all()
    else:
        assert (got[:cu[-1]] == ref[:cu[-1]]).all()


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
def test_group_gemm_operand_above_2gb(op):
    """An operand that extends more than 2 GB past a tile's start: its buffer resources count
    more bytes than a resource holds for the first K steps (the count saturates), then the
    exact remainder, down to the zero fill past the contraction's end.  The 2 GB operand is
    zero except for chosen rows (the first steps, the middle, the end), so the oracle needs
    only those; ternary values keep every sum exact.
      FWD:   W [1, 32768, 32776] (2.15 GB), nonzero contraction rows;
      DGRAD: W [1, 16384, 65544] (2.15 GB), nonzero output rows (columns of the result);
      WGRAD: a [262508, 4096] (2.15 GB), a 262444-row segment then a 64-row one, nonzero
             rows at the long segment's start and end and all of the short one (an over-read
             past the first segment's end would pick them up)."""
    m = mod()
    M = 300
    rng = np.random.default_rng(21)
    log(f"gemm operand above 2 GB op={op}")
    if op == "fwd":
        Kd, N = 32768, 32776
        nz = np.unique(np.concatenate([np.arange(0, 40), np.arange(16370, 16410),
                                       np.arange(Kd - 40, Kd), rng.integers(0, Kd, 100)]))
        a = synth.to_bf16_bits(synth.host_ternary(21, 1, (M, Kd)))
        w_nz = synth.to_bf16_bits(synth.host_ternary(21, 2, (nz.size, N)))
        W = torch.zeros((1, Kd, N), dtype=torch.bfloat16, device="cuda")
        W[0, torch.as_tensor(nz, device="cuda")] = from_bits(w_nz)
        cu = np.array([0, M], np.int32)
        out = poisoned((M, N), torch.bfloat16)
        m.moe_group_gemm(m.GEMM_FWD, from_bits(a), W, _dev(cu), out, Kd, N)
        got = bits(out)
        del W
        ref = oracle.group_gemm("fwd", np.ascontiguousarray(a[:, nz]), w_nz[None], cu, "bf16")
        assert (got == ref).all()
    elif op == "dgrad":
        Kd, N = 16384, 65544
        nz = np.unique(np.concatenate([np.arange(0, 64), np.arange(8000, 8064),
                                       np.arange(Kd - 64, Kd), rng.integers(0, Kd, 64)]))
        a = synth.to_bf16_bits(synth.host_ternary(21, 3, (M, N)))
        w_nz = synth.to_bf16_bits(synth.host_ternary(21, 4, (nz.size, N)))
        W = torch.zeros((1, Kd, N), dtype=torch.bfloat16, device="cuda")
        W[0, torch.as_tensor(nz, device="cuda")] = from_bits(w_nz)
        cu = np.array([0, M], np.int32)
        out = poisoned((M, Kd), torch.bfloat16)
        m.moe_group_gemm(m.GEMM_DGRAD, from_bits(a), W, _dev(cu), out, Kd, N)
        got = bits(out)
        del W
        ref = oracle.group_gemm("dgrad", a, w_nz[None], cu, "bf16")
        assert (got[:, nz] == ref).all()
        rest = np.setdiff1d(np.arange(Kd), nz)
        assert ((got[:, rest] & 0x7FFF) == 0).all(), "columns of zero weight rows are zero"
    else:
        Kd, N = 4096, 256
        L0, L1 = 262444, 64
        Mw = L0 + L1
        nz0 = np.unique(np.concatenate([np.arange(0, 400), np.arange(L0 - 44, L0),
                                        rng.integers(0, L0, 100)]))
        rows = np.concatenate([nz0, np.arange(L0, Mw)])
        a_nz = synth.to_bf16_bits(synth.host_ternary(21, 5, (rows.size, Kd)))
        A = torch.zeros((Mw, Kd), dtype=torch.bfloat16, device="cuda")
        A[torch.as_tensor(rows, device="cuda")] = from_bits(a_nz)
        b = synth.to_bf16_bits(synth.host_ternary(21, 6, (Mw, N)))
        cu = np.array([0, L0, Mw], np.int32)
        init = synth.host_ternary(21, 7, (2, Kd, N))
        out = _dev(init.astype(np.float32))
        m.moe_group_gemm(m.GEMM_WGRAD, A, from_bits(b), _dev(cu), out, Kd, N)
        got = out.cpu().numpy()
        del A
        cu_c = np.array([0, nz0.size, rows.size], np.int32)
        ref = oracle.group_gemm("wgrad", a_nz, np.ascontiguousarray(b[rows]), cu_c, "bf16",
                                out=init)
        assert (got == ref).all()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("op", ["fwd", "dgrad", "wgrad"])
def test_group_gemm_f32(op):
    G, M, Kd, N = 18, 256, 256, 512
    rng = np.random.default_rng(4)
    cu = _segments(rng, G, M)
    a, b = _gemm_inputs(op, G, M, Kd, N, "f32", lambda t, s: synth.host_normal(3, t, s))
    init = np.zeros((G, Kd, N), np.float32) if op == "wgrad" else None
    got = _run_gemm(op, a, b, cu, Kd, N, "f32", init)
    ref = oracle.group_gemm(op, a, b, cu, "f32", out=init)
    check_close(got, ref, "f32", what=f"f32 gemm {op}")


def test_group_gemm_deterministic():
    G, M, Kd, N = 9, 1500, 512, 768
    rng = np.random.default_rng(8)
    cu = _segments(rng, G, M)
    a, b = _gemm_inputs("fwd", G, M, Kd, N, "bf16", lambda t, s: synth.host_normal(1, t, s))
    r1 = _run_gemm("fwd", a, b, cu, Kd, N, "bf16")
    r2 = _run_gemm("fwd", a, b, cu, Kd, N, "bf16")
    assert (r1 == r2).all()


# ------------------------------------------------------------------------------------------
# tiny fp32 workload end to end (plan, permute, one projection, combine; rank 0)
# ------------------------------------------------------------------------------------------

def test_tiny_f32_workload_end_to_end():
    w = synth.WORKLOADS["tiny_f32"]
    d = w.dims
    idx, topk_w = synth.routing(d, w.zipf_s, w.base_seed)
    x = synth.host_normal(w.base_seed, 10, (d.R * d.S, d.H))
    W_up = synth.host_normal(w.base_seed, 11, (d.G, d.H, d.Hp), 0.02)
    Y_stage = synth.host_normal(w.base_seed, 12, (d.R * d.SK, d.Hp))
    rank = 0
    pl = oracle.plan(idx, d.E, d.B)
    assert pl.status == 0
    W_up = oracle.prefetch(W_up, pl, rank)   # the oracle's view of the slot rows
    m = mod()
    gp = GpuPlan(d.R, d.S, d.K, d.E, d.B)
    gp.run(_dev(idx), rank)
    check_plan_layout(gp, idx, rank, pl)
    Wd = _dev(synth.host_normal(w.base_seed, 11, (d.G, d.H, d.Hp), 0.02))
    m.moe_prefetch(gp.d, rank, gp.plan, Wd)
    assert (Wd.cpu().numpy() == W_up).all()
    xp = poisoned((d.SK, d.H), torch.float32)
    m.moe_permute(gp.d, _dev(x), gp.src, xp)
    Y = _dev(Y_stage)
    y_view = Y[rank * d.SK:(rank + 1) * d.SK]
    m.moe_group_gemm(m.GEMM_FWD, xp, Wd, gp.cu, y_view, d.H, d.Hp)
    out = poisoned((d.S, d.Hp), torch.float32)
    m.moe_combine(gp.d, rank, Y, gp.dest, _dev(topk_w.reshape(-1)), out)
    # oracle
    _, dest, src = oracle.layout(idx, pl, rank)
    cu = pl.cu_seqlens()[rank]
    xp_ref = oracle.permute(x, src, d.K, dtype="f32")
    assert (xp.cpu().numpy() == xp_ref).all()
    y_ref = oracle.group_gemm("fwd", xp_ref, W_up, cu, "f32")
    check_close(y_view.cpu().numpy(), y_ref, "f32", what="tiny up-projection")
    Y_ref = Y_stage.copy()
    Y_ref[rank * d.SK:(rank + 1) * d.SK] = y_ref
    out_ref = oracle.combine(Y_ref, dest, topk_w, rank, d.S, d.K, "f32")
    check_close(out.cpu().numpy(), out_ref, "f32", what="tiny combine")


# ------------------------------------------------------------------------------------------
# gated (SwiGLU) variant
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("G,M,Kd,N", [(5, 700, 64, 256), (6, 1000, 136, 400), (3, 2100, 520, 528),
                                      (9, 257, 1408, 4096)])
def test_group_gemm_swiglu(G, M, Kd, N):
    rng = np.random.default_rng(G * 1000 + N)
    m = mod()
    cu = _segments(rng, G, M)
    a = synth.to_bf16_bits(rng.standard_normal((M, Kd)).astype(np.float32))
    W = synth.to_bf16_bits((rng.standard_normal((G, Kd, N)) * (2.0 / np.sqrt(Kd))).astype(np.float32))
    z = poisoned((M, N // 2), torch.bfloat16)
    h = poisoned((M, N), torch.bfloat16)
    m.moe_group_gemm_swiglu(from_bits(a), from_bits(W), _dev(cu), z, h, Kd, N)
    z_ref, h_ref = oracle.group_gemm_swiglu(a, W, cu, "bf16")
    rows = np.arange(cu[0], cu[-1])
    check_close(bits(h)[rows], h_ref[rows], "bf16", what=f"swiglu pre-activation {G},{M},{Kd},{N}")
    # normwise bf16 tolerance as for every GEMM output: a per-element bound does not hold where
    # the gate or up pre-activation is a near-cancelling sum (fp32 vs float64 accumulation)
    check_close(bits(z)[rows], z_ref[rows], "bf16", min_identical=0.95,
                what=f"swiglu z {G},{M},{Kd},{N}")
    # z alone (no pre-activation output) gives the same z
    z2 = poisoned((M, N // 2), torch.bfloat16)
    m.moe_group_gemm_swiglu(from_bits(a), from_bits(W), _dev(cu), z2, None, Kd, N)
    assert (bits(z2)[rows] == bits(z)[rows]).all()


@pytest.mark.parametrize("Kd", [256, 224, 192, 160])
def test_group_gemm_swiglu_integer_preactivation(Kd):
    """On ternary inputs the pre-activation is exact, so it must match the oracle bit for bit.
    The gated kernel runs its K loop unrolled over the four ring stages with the last
    nk % 4 steps after the loop: Kd = 256, 224, 192, 160 give 8, 7, 6, 5 K steps (remainders
    0, 3, 2, 1)."""
    rng = np.random.default_rng(3)
    G, M, N = 4, 900, 512
    m = mod()
    cu = _segments(rng, G, M)
    a = synth.to_bf16_bits(synth.host_ternary(1, 1, (M, Kd)))
    W = synth.to_bf16_bits(synth.host_ternary(1, 2, (G, Kd, N)))
    z = poisoned((M, N // 2), torch.bfloat16)
    h = poisoned((M, N), torch.bfloat16)
    m.moe_group_gemm_swiglu(from_bits(a), from_bits(W), _dev(cu), z, h, Kd, N)
    z_ref, h_ref = oracle.group_gemm_swiglu(a, W, cu, "bf16")
    rows = np.arange(cu[0], cu[-1])
    assert (bits(h)[rows] == h_ref[rows]).all()
    # the pre-activation is exact here, so z differs from the oracle only by fp32 SiLU and
    # one rounding: within one bf16 unit in the last place everywhere
    within_one_bf16_ulp(bits(z)[rows], z_ref[rows], what="swiglu z on ternary inputs")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_swiglu_backward(dtype):
    rng = np.random.default_rng(11)
    M, Np = 1000, 264
    h = (rng.standard_normal((M, 2 * Np)) * 2.5).astype(np.float32)
    dz = rng.standard_normal((M, Np)).astype(np.float32)
    if dtype == "bf16":
        h, dz = synth.to_bf16_bits(h), synth.to_bf16_bits(dz)
    m = mod()
    dh = poisoned((M, 2 * Np), torch.bfloat16 if dtype == "bf16" else torch.float32)
    m.moe_swiglu_backward(from_bits(h), from_bits(dz), dh)
    ref = oracle.swiglu_backward(dz, h, dtype)
    check_close(bits(dh), ref, dtype, tol=2e-2 if dtype == "bf16" else 1e-5,
                min_identical=0.95, what=f"swiglu backward {dtype}")


def test_gated_layer_step_against_oracle():
    """Tiny gated layer on rank 0: dispatch, gated up, down, and the backward through the gated
    unit (down DGRAD, swiglu backward, up DGRAD, up WGRAD), each stage against the oracle's own
    chain from the generated inputs (no GPU output is fed to the oracle).  The chained stages
    carry the earlier stages' bf16 roundings, so they are checked normwise (2e-2) without a
    floor on bit-identical elements."""
    R, S, K, E, B, H, Hp = 4, 96, 2, 16, 2, 64, 48
    idx, pl = _plan_for(R, S, K, E, B, 33)
    m = mod()
    d = m.dims(R, S, K, E, B)
    G, SK, rank = E + B, S * K, 0
    cu, dest, src = oracle.layout(idx, pl, rank)
    rng = np.random.default_rng(4)
    x = synth.to_bf16_bits(rng.standard_normal((R * S, H)).astype(np.float32))
    Wu = synth.to_bf16_bits((rng.standard_normal((G, H, 2 * Hp)) * 0.25).astype(np.float32))
    Wd = synth.to_bf16_bits((rng.standard_normal((G, Hp, H)) * 0.25).astype(np.float32))
    dout = synth.to_bf16_bits(rng.standard_normal((R * S, H)).astype(np.float32))
    w = rng.random(R * S * K).astype(np.float32)
    Wu_d, Wd_d = from_bits(Wu), from_bits(Wd)
    plan_d = _dev(pl.to_blob())
    m.moe_prefetch(d, rank, plan_d, Wu_d)
    m.moe_prefetch(d, rank, plan_d, Wd_d)
    Wu_r, Wd_r = oracle.prefetch(Wu, pl, rank), oracle.prefetch(Wd, pl, rank)
    xp = poisoned((SK, H), torch.bfloat16)
    m.moe_permute(d, from_bits(x), _dev(src), xp)
    z = poisoned((SK, Hp), torch.bfloat16)
    hpre = poisoned((SK, 2 * Hp), torch.bfloat16)
    cu_d = _dev(cu)
    m.moe_group_gemm_swiglu(xp, Wu_d, cu_d, z, hpre, H, 2 * Hp)
    y = poisoned((SK, H), torch.bfloat16)
    m.moe_group_gemm(m.GEMM_FWD, z, Wd_d, cu_d, y, Hp, H)
    xp_r = oracle.permute(x, src, K)
    assert (bits(xp) == xp_r).all()
    z_r, h_r = oracle.group_gemm_swiglu(xp_r, Wu_r, cu, "bf16")
    check_close(bits(hpre), h_r, "bf16", what="gated layer pre-activation")
    check_close(bits(z), z_r, "bf16", min_identical=0.95, what="gated layer z")
    y_r = oracle.group_gemm("fwd", z_r, Wd_r, cu, "bf16")
    check_close(bits(y), y_r, "bf16", min_identical=0.0, what="gated layer down projection")
    dy = poisoned((SK, H), torch.bfloat16)
    m.moe_permute(d, from_bits(dout), _dev(src), dy, row_scale=_dev(w))
    dz = poisoned((SK, Hp), torch.bfloat16)
    m.moe_group_gemm(m.GEMM_DGRAD, dy, Wd_d, cu_d, dz, Hp, H)
    dh = poisoned((SK, 2 * Hp), torch.bfloat16)
    m.moe_swiglu_backward(hpre, dz, dh)
    dxp = poisoned((SK, H), torch.bfloat16)
    m.moe_group_gemm(m.GEMM_DGRAD, dh, Wu_d, cu_d, dxp, H, 2 * Hp)
    dWu = torch.zeros((G, H, 2 * Hp), dtype=torch.float32, device="cuda")
    m.moe_group_gemm(m.GEMM_WGRAD, xp, dh, cu_d, dWu, H, 2 * Hp)
    dy_r = oracle.permute(dout, src, K, row_scale=w)
    assert (bits(dy) == dy_r).all()
    dz_r = oracle.group_gemm("dgrad", dy_r, Wd_r, cu, "bf16")
    check_close(bits(dz), dz_r, "bf16", what="gated layer down dgrad")
    dh_r = oracle.swiglu_backward(dz_r, h_r, "bf16")
    check_close(bits(dh), dh_r, "bf16", min_identical=0.0, what="gated layer swiglu backward")
    dxp_r = oracle.group_gemm("dgrad", dh_r, Wu_r, cu, "bf16")
    check_close(bits(dxp), dxp_r, "bf16", min_identical=0.0, what="gated layer up dgrad")
    dWu_r = oracle.group_gemm("wgrad", xp_r, dh_r, cu, "bf16",
                              out=np.zeros((G, H, 2 * Hp), np.float32))
    # fp32 output, but its row operand dh went through the bf16 chain: the bf16 tolerance
    check_close(dWu.cpu().numpy(), dWu_r, "f32", tol=2e-2, min_identical=0.0,
                what="gated layer up wgrad")
