"""Full-size parity: every workload shape, the launch configuration bench.py times.

One forward + backward step of rank 0 runs call by call through the C ABI (via LayerStep).
Plan, counts, cu_seqlens, dest_pos and src_flat are compared with the oracle bit for bit
over the whole routing; the dense outputs are checked on sampled rows / tokens / weight
entries, each recomputed by the oracle from the generated inputs alone (x -> z -> y, dOut ->
dy -> dz -> dxp): no value the HIP path produced is ever fed to the oracle.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import check_close, log, router_grad_bound

pytestmark = pytest.mark.gpu


def host_rows(t, idx):
    idx = torch.as_tensor(np.asarray(idx, np.int64), device=t.device)
    r = t[idx]
    if r.dtype == torch.bfloat16:
        return r.view(torch.int16).cpu().numpy().view(np.uint16)
    return r.cpu().numpy()


class HostWeights:
    """Oracle view of a device weight tensor after prefetch: slot row E+j reads expert e."""

    def __init__(self, dev, pl, rank):
        self.dev = dev
        se, _, _ = pl.slot_table()
        self.map = {pl.E + j: int(se[rank, j]) for j in range(pl.B) if se[rank, j] >= 0}
        self.shape = tuple(dev.shape)
        self.cache = {}

    def __getitem__(self, rho):
        rho = int(rho)
        if rho not in self.cache:
            self.cache[rho] = host_rows(self.dev, [self.map.get(rho, rho)])[0]
        return self.cache[rho]


def sum_abs_products(y, dest, dout, rank, S, K, tokens):
    """[tokens, K]: sum_h |dout[s, h] * y[row of copy (rank, s, k), h]| of bf16 rows."""
    out = np.zeros((len(tokens), K))
    dp = np.asarray(dest).reshape(-1)
    for t, s_ in enumerate(tokens):
        g = np.abs(oracle.bf16_bits_to_f64(dout[int(s_)]))
        for k in range(K):
            dd = int(dp[(rank * S + int(s_)) * K + k])
            if dd >= 0:
                out[t, k] = float(np.dot(g, np.abs(oracle.bf16_bits_to_f64(y[dd]))))
    return out


def compact_cu(seg, G):
    counts = np.bincount(np.asarray(seg, np.int64), minlength=G)
    return np.concatenate([[0], np.cumsum(counts)])


WORKLOADS = [("balanced_bf16", None), ("skew1_large", 1.0), ("skew8_large_fwdbwd", 8.0),
             ("sweep_r64", 16.0), ("sweep_r64", 4.0), ("sweep_r64", 1.0), ("sweep_r64", 0.0)]


def seg_weight_cols(W, rho, cols):
    """[1, rows, len(cols)]: columns `cols` of weight row rho (a FWD over them gives exactly
    those output columns: every output element is its own float64 dot product)."""
    return W[rho][:, np.asarray(cols)][None]


def seg_weight_rows(W, rho, rows):
    """[1, len(rows), cols]: rows `rows` of weight row rho (a DGRAD over them gives exactly
    those output columns)."""
    return W[rho][np.asarray(rows)][None]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name,target", WORKLOADS)
def test_full_size_step(name, target):
    from balanced_token_dispatch_amd import (GEMM_DGRAD, GEMM_FWD, GEMM_WGRAD, moe_combine,
                                             moe_combine_weight_grad, moe_dispatch_layout,
                                             moe_group_gemm, moe_group_gemm_gather, moe_permute,
                                             moe_plan, moe_prefetch, moe_replica_grad_fold,
                                             moe_unpermute_reduce)
    from balanced_token_dispatch_amd.layer import LayerStep, Shape
    wl = synth.WORKLOADS[name]
    d = wl.dims
    rank = 0
    zipf = synth.zipf_for(wl, target)
    idx, w = synth.routing(d, zipf, wl.base_seed)
    log(f"full size {name} target={target} maxvio={synth.realised_maxvio(idx, d.E):.3f}")
    L = LayerStep(Shape(d.R, d.S, d.K, d.E, d.B, d.H, d.Hp), rank=rank)
    seed = wl.base_seed
    synth.fill_normal_(L.x_all, 1.0, seed * 10 + 1)
    synth.fill_normal_(L.w_up, 0.02, seed * 10 + 2)
    synth.fill_normal_(L.w_down, 0.02, seed * 10 + 3)
    synth.fill_normal_(L.y_all, 1.0, seed * 10 + 4)
    synth.fill_normal_(L.dout_all, 1.0, seed * 10 + 5)
    synth.fill_normal_(L.dxp_all, 1.0, seed * 10 + 6)   # the peers' slices; rank 0's is recomputed
    L.topk_idx.copy_(torch.from_numpy(idx))
    L.topk_w.copy_(torch.from_numpy(w))
    SK, S, K, E, B, H, Hp, G = d.SK, d.S, d.K, d.E, d.B, d.H, d.Hp, d.G
    rng = np.random.default_rng(seed)
    w_flat = w.reshape(-1)

    # --- plan + layout: bit-exact over the whole routing
    moe_plan(L.d, L.topk_idx, L.counts, L.plan, L.status, L.ws)
    moe_dispatch_layout(L.d, rank, L.topk_idx, L.plan, L.cu, L.dest, L.src, L.ws)
    torch.cuda.synchronize()
    pl = oracle.plan(idx, E, B)
    assert pl.status == 0, "no overflow at the workload shapes"
    assert (L.plan.cpu().numpy() == pl.to_blob()).all()
    assert (L.counts.cpu().numpy() == pl.counts).all()
    cu, dest, src = oracle.layout(idx, pl, rank)
    assert (L.cu.cpu().numpy() == cu).all()
    assert (L.dest.cpu().numpy() == dest).all()
    assert (L.src.cpu().numpy() == src).all()
    assert cu[-1] == SK
    log(f"  plan+layout exact; replicas={len(pl.replicas)} max/rank={pl.max_needed}")

    # --- prefetch: each used slot row is a bitwise copy of its expert
    w_up0 = L.w_up.clone() if G * H * Hp * 2 < 12e9 else None
    moe_prefetch(L.d, rank, L.plan, L.w_up)
    moe_prefetch(L.d, rank, L.plan, L.w_down)
    se, _, _ = pl.slot_table()
    for j in range(B):
        e = int(se[rank, j])
        if e >= 0:
            assert torch.equal(L.w_up[E + j], L.w_up[e]) and torch.equal(L.w_down[E + j], L.w_down[e])
    if w_up0 is not None:
        assert torch.equal(L.w_up[:E], w_up0[:E]), "home rows untouched"
        del w_up0

    Wu, Wd = HostWeights(L.w_up, pl, rank), HostWeights(L.w_down, pl, rank)
    # sampled buffer rows: the first and last row of every active segment plus random rows,
    # restricted to a few segments so the oracle fetches few weight rows
    act = [rho for rho in range(G) if cu[rho + 1] > cu[rho]]
    pick = sorted(set(rng.choice(act, size=min(3, len(act)), replace=False).tolist())
                  | {act[-1]})
    rows = []
    for rho in pick:
        lo, hi = int(cu[rho]), int(cu[rho + 1])
        rows += [lo, hi - 1] + rng.integers(lo, hi, size=10).tolist()
    rows = np.array(sorted(set(rows)), np.int64)
    seg = np.searchsorted(cu, rows, side="right") - 1
    cu_c = compact_cu(seg, G)
    toks = src[rows] // K

    # --- forward: permute, up, down, combine
    moe_permute(L.d, L.x_all, L.src, L.xp)
    moe_group_gemm(GEMM_FWD, L.xp, L.w_up, L.cu, L.z, H, Hp, L.gemm_ws)
    moe_group_gemm(GEMM_FWD, L.z, L.w_down, L.cu, L.y, Hp, H, L.gemm_ws)
    moe_combine(L.d, rank, L.y_all, L.dest, L.topk_w.view(-1), L.out)
    torch.cuda.synchronize()
    x_rows = host_rows(L.x_all, toks)
    assert (host_rows(L.xp, rows) == x_rows).all(), "permute rows"
    _, z_ref = oracle.group_gemm_rows("fwd", x_rows, Wu, cu_c, np.arange(rows.size))
    check_close(host_rows(L.z, rows), z_ref, "bf16", what="up projection rows")
    # the permute fused into the up projection: the same bits as permute + GEMM, every row
    z_g = torch.empty_like(L.z)
    moe_group_gemm_gather(GEMM_FWD, L.x_all, L.src, K, L.w_up, L.cu, z_g, H, Hp, L.gemm_ws)
    torch.cuda.synchronize()
    assert torch.equal(z_g.view(torch.int16), L.z.view(torch.int16)), "gathered up projection"
    check_close(host_rows(z_g, rows), z_ref, "bf16", what="gathered up projection rows")
    del z_g
    _, y_ref = oracle.group_gemm_rows("fwd", z_ref, Wd, cu_c, np.arange(rows.size))
    check_close(host_rows(L.y, rows), y_ref, "bf16", what="down projection rows")
    # combine: tokens whose copies landing on rank 0 are all in the sampled segments
    tok_s = []
    for s_ in rng.permutation(S)[:4096]:
        ds = dest[(rank * S + s_) * K:(rank * S + s_ + 1) * K]
        mine = ds[(ds >= rank * SK) & (ds < (rank + 1) * SK)] - rank * SK
        if np.isin(np.searchsorted(cu, mine, side="right") - 1, pick).all():
            tok_s.append(int(s_))
        if len(tok_s) == 12:
            break
    if len(tok_s) < 2:
        tok_s = sorted(set(tok_s) | {0, S - 1})
    need = dest.reshape(d.R, S, K)[rank, tok_s].reshape(-1)
    y_tab = host_rows(L.y_all, need)          # staged rows of other ranks: generated inputs
    for k_, dd in enumerate(need):             # rank-0 rows: the oracle's own chain
        if rank * SK <= dd < (rank + 1) * SK:
            r_ = dd - rank * SK
            rho = int(np.searchsorted(cu, r_, side="right") - 1)
            xr = host_rows(L.x_all, [src[r_] // K])
            cu1 = compact_cu([rho], G)
            _, zr = oracle.group_gemm_rows("fwd", xr, Wu, cu1, [0])
            _, yr = oracle.group_gemm_rows("fwd", zr, Wd, cu1, [0])
            y_tab[k_] = yr[0]
    copies = ((rank * S + np.array(tok_s))[:, None] * K + np.arange(K)[None, :]).reshape(-1)
    dest_l = np.full(dest.size, -1, np.int64)
    dest_l[copies] = np.arange(copies.size)          # need[i] is the row of copies[i]
    out_ref = oracle.combine(y_tab, dest_l, w, rank, S, K, "bf16", tokens=tok_s)
    check_close(host_rows(L.out, tok_s), out_ref, "bf16", what="combine tokens")
    # and up to 128 tokens none of whose copies lands on rank 0: every row they gather is a
    # peer's staged row (a generated input)
    dest3 = dest.reshape(d.R, S, K)[rank]
    far = np.flatnonzero(((dest3 >= rank * SK) & (dest3 < (rank + 1) * SK)).sum(axis=1) == 0)
    tok_z = np.sort(rng.permutation(far)[:128]).tolist()
    need_z = dest3[tok_z].reshape(-1)
    copies_z = ((rank * S + np.array(tok_z, np.int64))[:, None] * K
                + np.arange(K)[None, :]).reshape(-1)
    dest_z = np.full(dest.size, -1, np.int64)
    dest_z[copies_z] = np.where(need_z >= 0, np.arange(copies_z.size), -1)
    yz = host_rows(L.y_all, np.maximum(need_z, 0))
    out_z = oracle.combine(yz, dest_z, w, rank, S, K, "bf16", tokens=tok_z)
    check_close(host_rows(L.out, tok_z), out_z, "bf16", what="combine, tokens gathering staged rows")
    log(f"  forward sampled rows within tolerance; combine of {len(tok_s)} + {len(tok_z)} tokens")

    # --- backward: weighted permute, down dgrad/wgrad, up dgrad/wgrad, fold
    moe_permute(L.d, L.dout_all, L.src, L.dy, L.topk_w.view(-1))
    moe_group_gemm(GEMM_DGRAD, L.dy, L.w_down, L.cu, L.dz, Hp, H, L.gemm_ws)
    L.dw_down.zero_()
    L.dw_up.zero_()
    moe_group_gemm(GEMM_WGRAD, L.z, L.dy, L.cu, L.dw_down, Hp, H)
    moe_group_gemm(GEMM_DGRAD, L.dz, L.w_up, L.cu, L.dxp, H, Hp, L.gemm_ws)
    moe_group_gemm(GEMM_WGRAD, L.xp, L.dz, L.cu, L.dw_up, H, Hp)
    dw_up_g = torch.zeros_like(L.dw_up)
    moe_group_gemm_gather(GEMM_WGRAD, L.x_all, L.src, K, L.dz, L.cu, dw_up_g, H, Hp)
    torch.cuda.synchronize()
    assert torch.equal(dw_up_g.view(torch.int32), L.dw_up.view(torch.int32)), "gathered up wgrad"
    g_rows = host_rows(L.dout_all, toks)
    src_l = (np.arange(rows.size) * K + src[rows] % K).astype(np.int32)   # compact copy ids
    rs = np.zeros(rows.size * K, np.float32)
    rs[src_l] = w_flat[src[rows]]
    dy_ref = oracle.permute(g_rows, src_l, K, row_scale=rs)
    assert (host_rows(L.dy, rows) == dy_ref).all(), "weighted permute rows"
    _, dz_ref = oracle.group_gemm_rows("dgrad", dy_ref, Wd, cu_c, np.arange(rows.size))
    check_close(host_rows(L.dz, rows), dz_ref, "bf16", what="down dgrad rows")
    _, dxp_ref = oracle.group_gemm_rows("dgrad", dz_ref, Wu, cu_c, np.arange(rows.size))
    check_close(host_rows(L.dxp, rows), dxp_ref, "bf16", what="up dgrad rows")
    # wgrad entries of the smallest sampled segment, at any segment length: an entry
    # dW_down[i, j] = sum_m z[m, i] dy[m, j] needs column i of z (x @ W_up[:, i]) and column j
    # of dy over the segment's rows; dW_up[i, j] = sum_m x[m, i] dz[m, j] needs column j of dz
    # (dy @ W_down[j, :]^T).  The oracle recomputes only those columns.
    rho = min(pick, key=lambda r_: cu[r_ + 1] - cu[r_])
    lo, hi = int(cu[rho]), int(cu[rho + 1])
    n_seg = hi - lo
    seg_rows = np.arange(lo, hi)
    stoks = src[seg_rows] // K
    xs = host_rows(L.x_all, stoks)
    gs = host_rows(L.dout_all, stoks)
    wsc = w_flat[src[seg_rows]]
    dys = oracle.permute(gs, (np.arange(n_seg) * K).astype(np.int32), K,
                         row_scale=np.repeat(wsc, K).astype(np.float32))
    cu2 = np.array([0, n_seg])
    ii = rng.integers(0, Hp, 8)
    jj = rng.integers(0, H, 8)
    z_cols = oracle.group_gemm("fwd", xs, seg_weight_cols(Wu, rho, ii), cu2, "bf16")
    ent = oracle.wgrad_entries(z_cols, dys, cu2, 0, np.arange(ii.size), jj, "bf16")
    got = L.dw_down[rho][torch.as_tensor(ii, device="cuda"),
                         torch.as_tensor(jj, device="cuda")].cpu().numpy()
    assert np.abs(got - ent).max() <= 1e-3 * max(1.0, np.abs(ent).max()), (got, ent)
    ii2 = rng.integers(0, H, 8)
    jj2 = rng.integers(0, Hp, 8)
    dz_cols = oracle.group_gemm("dgrad", dys, seg_weight_rows(Wd, rho, jj2), cu2, "bf16")
    ent2 = oracle.wgrad_entries(xs, dz_cols, cu2, 0, ii2, np.arange(jj2.size), "bf16")
    got2 = L.dw_up[rho][torch.as_tensor(ii2, device="cuda"),
                        torch.as_tensor(jj2, device="cuda")].cpu().numpy()
    assert np.abs(got2 - ent2).max() <= 1e-3 * max(1.0, np.abs(ent2).max()), (got2, ent2)
    got3 = dw_up_g[rho][torch.as_tensor(ii2, device="cuda"),
                        torch.as_tensor(jj2, device="cuda")].cpu().numpy()
    assert np.abs(got3 - ent2).max() <= 1e-3 * max(1.0, np.abs(ent2).max()), (got3, ent2)
    del dw_up_g
    log(f"  wgrad entries of segment {rho} ({n_seg} rows) within tolerance (also gathered)")
    # router-weight gradient and un-permute reduce.  Tokens none of whose copies lands on rank
    # 0 read only the peers' staged rows (generated inputs): the oracle takes those rows and the
    # GPU must match it within the summation bound.  The sampled tokens with copies on rank 0
    # read rank 0's expert outputs and input gradients, which the oracle recomputes by its own
    # chain (x -> z -> y above; dOut -> dy -> dz -> dxp here); the GPU's chain rounds those rows
    # on its own, so there the check is normwise.
    moe_combine_weight_grad(L.d, rank, L.y_all, L.dest, L.dout_all[rank * S:(rank + 1) * S],
                            L.dtopk_w)
    moe_unpermute_reduce(L.d, rank, L.dxp_all, L.dest, L.dx)
    torch.cuda.synchronize()
    dw_all = L.dtopk_w.view(S, K)
    # (a) staged rows only
    gz = np.zeros((S, H), np.uint16)
    gz[tok_z] = host_rows(L.dout_all, rank * S + np.array(tok_z))
    dwz_ref = oracle.combine_weight_grad(yz, dest_z, gz, rank, S, K, "bf16", tokens=tok_z)
    dwz_got = dw_all[torch.as_tensor(tok_z, device="cuda")].cpu().numpy()
    bound = router_grad_bound(yz, dest_z, gz, rank, S, K, "bf16", H, tokens=tok_z)
    err = np.abs(dwz_got.astype(np.float64) - dwz_ref.astype(np.float64))
    assert (err <= bound + np.abs(dwz_ref) * 2.0 ** -24).all(), "router-weight gradient, staged rows"
    dxz_ref = oracle.unpermute_reduce(host_rows(L.dxp_all, np.maximum(need_z, 0)), dest_z, rank,
                                      S, K, "bf16", tokens=tok_z)
    check_close(host_rows(L.dx, tok_z), dxz_ref, "bf16", what="un-permute reduce, staged rows")
    # (b) tokens with copies on rank 0, rank 0's rows from the oracle's chain
    dxp_tab = host_rows(L.dxp_all, need)       # staged rows of other ranks: generated inputs
    for k_, dd in enumerate(need):
        if rank * SK <= dd < (rank + 1) * SK:
            r_ = dd - rank * SK
            rho = int(np.searchsorted(cu, r_, side="right") - 1)
            gr = host_rows(L.dout_all, [src[r_] // K])
            dyr = oracle.permute(gr, np.array([src[r_] % K], np.int32), K,
                                 row_scale=np.where(np.arange(K) == src[r_] % K,
                                                    w_flat[src[r_]], 0).astype(np.float32))
            cu1 = compact_cu([rho], G)
            _, dzr = oracle.group_gemm_rows("dgrad", dyr, Wd, cu1, [0])
            _, dxr = oracle.group_gemm_rows("dgrad", dzr, Wu, cu1, [0])
            dxp_tab[k_] = dxr[0]
    g_full = np.zeros((S, H), np.uint16)
    g_full[tok_s] = host_rows(L.dout_all, rank * S + np.array(tok_s))
    dw_ref = oracle.combine_weight_grad(y_tab, dest_l, g_full, rank, S, K, "bf16", tokens=tok_s)
    dw_got = dw_all[torch.as_tensor(tok_s, device="cuda")].cpu().numpy()
    # the GPU's y rows on rank 0 may differ from the oracle's by one bf16 unit (at most 2^-7
    # of the value) in any element
    gy = sum_abs_products(y_tab, dest_l, g_full, rank, S, K, tok_s)
    bound = router_grad_bound(y_tab, dest_l, g_full, rank, S, K, "bf16", H, tokens=tok_s)
    err = np.abs(dw_got.astype(np.float64) - dw_ref.astype(np.float64))
    assert (err <= bound + gy * 2.0 ** -7).all(), (dw_got, dw_ref)
    dx_ref = oracle.unpermute_reduce(dxp_tab, dest_l, rank, S, K, "bf16", tokens=tok_s)
    check_close(host_rows(L.dx, tok_s), dx_ref, "bf16", min_identical=0.0,
                what="un-permute reduce tokens")
    log(f"  router-weight gradient and un-permute reduce of {len(tok_z)} + {len(tok_s)} tokens "
        f"within tolerance")
    # fold: home rows gain the slot rows, slot rows end zero (bitwise, on a sampled column block)
    cols = slice(0, 4096)
    before = {int(e): (L.dw_up[e].view(-1)[cols].cpu().numpy(),
                       L.dw_up[E + j].view(-1)[cols].cpu().numpy())
              for j, e in enumerate(se[rank]) if e >= 0}
    moe_replica_grad_fold(L.d, rank, L.plan, L.dw_up)
    torch.cuda.synchronize()
    for j, e in enumerate(se[rank]):
        if e < 0:
            continue
        h0, s0 = before[int(e)]
        assert (L.dw_up[e].view(-1)[cols].cpu().numpy() == h0 + s0).all()
        assert not L.dw_up[E + j].any()
    log(f"  backward sampled rows within tolerance; folded {len(before)} slot rows")
    del L
    gc.collect()
    torch.cuda.empty_cache()


def test_full_size_gated_step():
    """The gated layer at the headline shape (H=7168, H'=2048, up projection 7168 x 4096),
    run as the benchmark runs it (LayerStep.forward + backward, activation="swiglu"); the
    pre-activation, z, y, dz, dh, dxp rows and up-WGRAD entries are checked on sampled rows,
    each recomputed by the oracle from the generated inputs alone."""
    from balanced_token_dispatch_amd.layer import LayerStep, Shape
    wl = synth.WORKLOADS["skew8_large_fwdbwd"]
    d = wl.dims
    rank = 0
    idx, w = synth.routing(d, synth.zipf_for(wl, 8.0), wl.base_seed)
    log(f"full size gated step maxvio={synth.realised_maxvio(idx, d.E):.3f}")
    L = LayerStep(Shape(d.R, d.S, d.K, d.E, d.B, d.H, d.Hp), rank=rank, activation="swiglu")
    seed = wl.base_seed
    synth.fill_normal_(L.x_all, 1.0, seed * 10 + 1)
    synth.fill_normal_(L.w_up, 0.02, seed * 10 + 2)
    synth.fill_normal_(L.w_down, 0.02, seed * 10 + 3)
    synth.fill_normal_(L.y_all, 1.0, seed * 10 + 4)
    synth.fill_normal_(L.dout_all, 1.0, seed * 10 + 5)
    synth.fill_normal_(L.dxp_all, 1.0, seed * 10 + 6)
    L.topk_idx.copy_(torch.from_numpy(idx))
    L.topk_w.copy_(torch.from_numpy(w))
    SK, S, K, E, B, H, Hp, G = d.SK, d.S, d.K, d.E, d.B, d.H, d.Hp, d.G
    L.forward()
    L.dw_up.zero_()
    L.dw_down.zero_()
    L.backward()
    torch.cuda.synchronize()
    pl = oracle.plan(idx, E, B)
    cu, dest, src = oracle.layout(idx, pl, rank)
    assert (L.cu.cpu().numpy() == cu).all() and (L.src.cpu().numpy() == src).all()
    Wu, Wd = HostWeights(L.w_up, pl, rank), HostWeights(L.w_down, pl, rank)
    assert Wu.shape == (G, H, 2 * Hp)
    se, _, _ = pl.slot_table()
    homes = {int(e) for e in se[rank] if e >= 0}
    rng = np.random.default_rng(seed + 1)
    act = [rho for rho in range(G) if cu[rho + 1] > cu[rho]]
    slots = [rho for rho in act if rho >= E]
    plain = [rho for rho in act if rho < E and rho not in homes]
    pick = sorted(set(rng.choice(plain, size=min(2, len(plain)), replace=False).tolist())
                  | set(slots[:1]))
    rows = []
    for rho in pick:
        lo, hi = int(cu[rho]), int(cu[rho + 1])
        rows += [lo, hi - 1] + rng.integers(lo, hi, size=4).tolist()
    rows = np.array(sorted(set(rows)), np.int64)
    seg = np.searchsorted(cu, rows, side="right") - 1
    cu_c = compact_cu(seg, G)
    toks = src[rows] // K
    x_rows = host_rows(L.x_all, toks)
    z_ref, h_ref = oracle.group_gemm_swiglu(x_rows, Wu, cu_c, "bf16")
    check_close(host_rows(L.hpre, rows), h_ref, "bf16", what="gated pre-activation rows")
    check_close(host_rows(L.z, rows), z_ref, "bf16", min_identical=0.95, what="gated z rows")
    _, y_ref = oracle.group_gemm_rows("fwd", z_ref, Wd, cu_c, np.arange(rows.size))
    check_close(host_rows(L.y, rows), y_ref, "bf16", what="down projection rows (gated)")
    g_rows = host_rows(L.dout_all, toks)
    src_l = (np.arange(rows.size) * K + src[rows] % K).astype(np.int32)
    rs = np.zeros(rows.size * K, np.float32)
    rs[src_l] = w.reshape(-1)[src[rows]]
    dy_ref = oracle.permute(g_rows, src_l, K, row_scale=rs)
    assert (host_rows(L.dy, rows) == dy_ref).all(), "weighted permute rows"
    _, dz_ref = oracle.group_gemm_rows("dgrad", dy_ref, Wd, cu_c, np.arange(rows.size))
    check_close(host_rows(L.dz, rows), dz_ref, "bf16", what="down dgrad rows (gated)")
    dh_ref = oracle.swiglu_backward(dz_ref, h_ref, "bf16")
    # dh compounds the last-place differences of dz, gate and up: fewer identical elements
    check_close(host_rows(L.dh, rows), dh_ref, "bf16", min_identical=0.85,
                what="gated backward rows")
    _, dxp_ref = oracle.group_gemm_rows("dgrad", dh_ref, Wu, cu_c, np.arange(rows.size))
    # its input dh already differs in the last place from the GPU's in up to 15% of elements,
    # so the rounded sums agree less often; the normwise bound is the same
    check_close(host_rows(L.dxp, rows), dxp_ref, "bf16", min_identical=0.95,
                what="up dgrad rows (gated)")
    log(f"  gated forward/backward rows within tolerance ({rows.size} rows, segments {pick})")
    # up-WGRAD entries of the smallest sampled home-expert segment (no fold touches it), at any
    # segment length: entry (i, c) of dW_up needs column c of dh, which needs the (gate, up)
    # pair p = c // 2 of the pre-activation (columns 2p, 2p+1 of x @ W_up) and column p of dz
    # (dy @ W_down[p, :]^T).  The oracle recomputes only those columns.
    rho = min([r_ for r_ in pick if r_ < E], key=lambda r_: cu[r_ + 1] - cu[r_])
    lo, hi = int(cu[rho]), int(cu[rho + 1])
    n_seg = hi - lo
    seg_rows = np.arange(lo, hi)
    stoks = src[seg_rows] // K
    xs = host_rows(L.x_all, stoks)
    gs = host_rows(L.dout_all, stoks)
    dys = oracle.permute(gs, (np.arange(n_seg) * K).astype(np.int32), K,
                         row_scale=np.repeat(w.reshape(-1)[src[seg_rows]], K).astype(np.float32))
    cu2 = np.array([0, n_seg])
    ii = rng.integers(0, H, 8)
    jj = rng.integers(0, 2 * Hp, 8)
    pairs = jj // 2
    hcols = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)   # gate, up of each pair
    hs = oracle.group_gemm("fwd", xs, Wu[rho][:, hcols][None], cu2, "bf16")
    dzs = oracle.group_gemm("dgrad", dys, Wd[rho][pairs][None], cu2, "bf16")
    dhs = oracle.swiglu_backward(dzs, hs, "bf16")                        # [n, 2 * len(jj)]
    sel = 2 * np.arange(jj.size) + (jj % 2)                              # column jj of dh
    ent = oracle.wgrad_entries(xs, dhs, cu2, 0, ii, sel, "bf16")
    got = L.dw_up[rho][torch.as_tensor(ii, device="cuda"),
                       torch.as_tensor(jj, device="cuda")].cpu().numpy()
    assert np.abs(got - ent).max() <= 1e-3 * max(1.0, np.abs(ent).max()), (got, ent)
    log(f"  gated up-WGRAD entries of segment {rho} ({n_seg} rows) within tolerance")
    del L
    gc.collect()
    torch.cuda.empty_cache()
