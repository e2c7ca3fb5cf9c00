"""The oracle's whole layer, simulated on every rank, vs the dense MoE definition.

Pins permute, group_gemm (fwd, dgrad, wgrad), combine, prefetch,
replica_grad_fold, unpermute_reduce and combine_weight_grad together:
whatever plan is chosen, every copy must be processed by (a copy of) its own
expert and come back to its token with its router weight (ainovat article,
invariant and mechanism paragraphs; blog "Real-World Use"), every replica's
weight gradient must end up in its home expert, and the gradients of the
token rows and of the router weights must be those of the dense layer.  With small-integer inputs every float64 product and sum is
exact, so the simulation and the dense definition must agree bit for bit.

The dense definition below is written independently of the oracle: one
token copy at a time, no plan, no layout.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits


def _rnd(x64, dtype):
    return f64_to_bf16_bits(x64) if dtype == "bf16" else x64.astype(np.float32)


def _wid(x, dtype):
    return bf16_bits_to_f64(x) if dtype == "bf16" else np.asarray(x, np.float64)


def dense_forward(x, idx, w, W_up, W_down, dtype):
    """out[t] = round(sum_k w[t,k] * round(round(x[t] @ Wup[e]) @ Wdown[e])), e = idx[t,k]."""
    RS, K = idx.shape[0] * idx.shape[1], idx.shape[2]
    flat_idx = idx.reshape(RS, K)
    flat_w = w.reshape(RS, K)
    out = np.zeros((RS, W_down.shape[2]), np.float64)
    for t in range(RS):
        for k in range(K):
            e = flat_idx[t, k]
            z = _rnd(_wid(x[t], dtype) @ _wid(W_up[e], dtype), dtype)
            y = _rnd(_wid(z, dtype) @ _wid(W_down[e], dtype), dtype)
            out[t] += np.float64(flat_w[t, k]) * _wid(y, dtype)
    return _rnd(out, dtype)


def dense_weight_grads(x, idx, w, W_up, W_down, dout, dtype):
    """Per-expert dW_up, dW_down summed over every copy routed to that expert (float64)."""
    RS, K = idx.shape[0] * idx.shape[1], idx.shape[2]
    E = W_up.shape[0]
    gu = np.zeros(W_up.shape, np.float64)
    gd = np.zeros(W_down.shape, np.float64)
    fi, fw = idx.reshape(RS, K), w.reshape(RS, K)
    for t in range(RS):
        for k in range(K):
            e = fi[t, k]
            xt = _wid(x[t], dtype)
            z = _rnd(xt @ _wid(W_up[e], dtype), dtype)
            dy = _rnd(np.float32(fw[t, k]) * _wid(dout[t], dtype).astype(np.float32), dtype)
            dz = _rnd(_wid(dy, dtype) @ _wid(W_down[e], dtype).T, dtype)
            gd[e] += np.outer(_wid(z, dtype), _wid(dy, dtype))
            gu[e] += np.outer(xt, _wid(dz, dtype))
    return gu, gd


def dense_input_and_router_grads(x, idx, w, W_up, W_down, dout, dtype):
    """dx[t] = round(sum_k dxp_k), dxp_k the copy's input gradient; dw[t,k] = <dout[t], y_k>."""
    RS, K = idx.shape[0] * idx.shape[1], idx.shape[2]
    fi, fw = idx.reshape(RS, K), w.reshape(RS, K)
    dx = np.zeros((RS, W_up.shape[1]), np.float64)
    dw = np.zeros((RS, K), np.float64)
    for t in range(RS):
        for k in range(K):
            e = fi[t, k]
            z = _rnd(_wid(x[t], dtype) @ _wid(W_up[e], dtype), dtype)
            y = _rnd(_wid(z, dtype) @ _wid(W_down[e], dtype), dtype)
            dw[t, k] = float(np.dot(_wid(dout[t], dtype), _wid(y, dtype)))
            dy = _rnd(np.float32(fw[t, k]) * _wid(dout[t], dtype).astype(np.float32), dtype)
            dz = _rnd(_wid(dy, dtype) @ _wid(W_down[e], dtype).T, dtype)
            dx[t] += _wid(_rnd(_wid(dz, dtype) @ _wid(W_up[e], dtype).T, dtype), dtype)
    return _rnd(dx, dtype), dw.astype(np.float32)


def simulate(dims, idx, w, x, W_up, W_down, dout, dtype):
    R, E, B, SK = dims.R, dims.E, dims.B, dims.SK
    pl = oracle.plan(idx, E, B)
    assert pl.status == 0
    G = E + B
    Hp, H = dims.Hp, dims.H
    # weight tensors with B empty slot rows appended
    Wu = np.concatenate([W_up, np.zeros((B,) + W_up.shape[1:], W_up.dtype)])
    Wd = np.concatenate([W_down, np.zeros((B,) + W_down.shape[1:], W_down.dtype)])
    Y_all = np.zeros((R * SK, H), W_up.dtype)
    per_rank = []
    dest_ref = None
    for q in range(R):
        cu, dest, src = oracle.layout(idx, pl, q)
        dest_ref = dest if dest_ref is None else dest_ref
        Wu_q, Wd_q = oracle.prefetch(Wu, pl, q), oracle.prefetch(Wd, pl, q)
        xp = oracle.permute(x, src, dims.K, dtype=dtype)
        z = oracle.group_gemm("fwd", xp, Wu_q, cu, dtype)
        y = oracle.group_gemm("fwd", z, Wd_q, cu, dtype)
        Y_all[q * SK:(q + 1) * SK] = y
        per_rank.append((cu, src, xp, z, Wu_q, Wd_q))
    outs = [oracle.combine(Y_all, dest_ref, w, r, dims.S, dims.K, dtype) for r in range(R)]
    out = np.concatenate(outs)
    # backward on every rank, then fold each rank's replica rows home
    gu_tot = np.zeros((E,) + W_up.shape[1:], np.float64)
    gd_tot = np.zeros((E,) + W_down.shape[1:], np.float64)
    DXP_all = np.zeros((R * SK, H), W_up.dtype)
    for q in range(R):
        cu, src, xp, z, Wu_q, Wd_q = per_rank[q]
        dy = oracle.permute(dout, src, dims.K, row_scale=w.reshape(-1), dtype=dtype)
        dz = oracle.group_gemm("dgrad", dy, Wd_q, cu, dtype)
        dWd = oracle.group_gemm("wgrad", z, dy, cu, dtype, out=np.zeros((G, Hp, H), np.float32))
        dxp = oracle.group_gemm("dgrad", dz, Wu_q, cu, dtype)
        assert dxp.shape == xp.shape
        DXP_all[q * SK:(q + 1) * SK] = dxp
        dWu = oracle.group_gemm("wgrad", xp, dz, cu, dtype, out=np.zeros((G, H, Hp), np.float32))
        dWu = oracle.replica_grad_fold(dWu, pl, q)
        dWd = oracle.replica_grad_fold(dWd, pl, q)
        assert not dWu[E:].any() and not dWd[E:].any(), "fold clears the slot rows"
        gu_tot += dWu[:E]
        gd_tot += dWd[:E]
    dx = np.concatenate([oracle.unpermute_reduce(DXP_all, dest_ref, r, dims.S, dims.K, dtype)
                         for r in range(R)])
    dw = np.concatenate([oracle.combine_weight_grad(Y_all, dest_ref,
                                                    dout[r * dims.S:(r + 1) * dims.S], r,
                                                    dims.S, dims.K, dtype) for r in range(R)])
    return pl, out, gu_tot, gd_tot, dx, dw


def _int_inputs(dims, seed, dtype):
    R, S, K, E = dims.R, dims.S, dims.K, dims.E
    idx, _ = synth.routing(dims, zipf_s=1.2, base_seed=seed)
    rng = np.random.default_rng(seed)
    w = rng.choice(np.array([0.25, 0.5, 1.0], np.float32), size=(R, S, K))
    x = synth.host_ternary(seed, 1, (R * S, dims.H))
    Wu = synth.host_ternary(seed, 2, (E, dims.H, dims.Hp))
    Wd = synth.host_ternary(seed, 3, (E, dims.Hp, dims.H))
    dout = synth.host_ternary(seed, 4, (R * S, dims.H))
    if dtype == "bf16":
        x, Wu, Wd, dout = (synth.to_bf16_bits(a) for a in (x, Wu, Wd, dout))
    return idx, w, x, Wu, Wd, dout


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_simulation_equals_dense_moe(dtype, seed):
    dims = synth.Dims(R=4, S=12, K=2, E=8, B=3, H=16, Hp=24)
    idx, w, x, Wu, Wd, dout = _int_inputs(dims, seed, dtype)
    pl, out, gu, gd, dx, dw = simulate(dims, idx, w, x, Wu, Wd, dout, dtype)
    assert len(pl.replicas) > 0, "the skewed routing must exercise replicas"
    ref = dense_forward(x, idx, w, Wu, Wd, dtype)
    assert (out == ref).all()
    gu_ref, gd_ref = dense_weight_grads(x, idx, w, Wu, Wd, dout, dtype)
    assert (gu == gu_ref).all() and (gd == gd_ref).all()
    dx_ref, dw_ref = dense_input_and_router_grads(x, idx, w, Wu, Wd, dout, dtype)
    assert (dx == dx_ref).all()
    assert (dw == dw_ref).all()
    assert np.abs(dw).sum() > 0 and np.abs(_wid(dx, dtype)).sum() > 0, "non-trivial gradients"


def test_group_gemm_matches_triple_loop():
    """Second tier: per-element loops on a tiny grouped GEMM (fwd, dgrad, wgrad), fp32."""
    rng = np.random.default_rng(5)
    G, Kd, N = 4, 3, 5
    cu = np.array([0, 2, 2, 5, 6])
    M = 7
    a = rng.standard_normal((M, Kd)).astype(np.float32)
    W = rng.standard_normal((G, Kd, N)).astype(np.float32)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    fwd = oracle.group_gemm("fwd", a, W, cu, "f32")
    dgr = oracle.group_gemm("dgrad", dy, W, cu, "f32")
    wgr = oracle.group_gemm("wgrad", a, dy, cu, "f32", out=np.ones((G, Kd, N), np.float32))
    for rho in range(G):
        for m in range(cu[rho], cu[rho + 1]):
            for n in range(N):
                s = sum(float(a[m, c]) * float(W[rho, c, n]) for c in range(Kd))
                assert fwd[m, n] == np.float32(s)
            for c in range(Kd):
                s = sum(float(dy[m, n]) * float(W[rho, c, n]) for n in range(N))
                assert dgr[m, c] == np.float32(s)
        for c in range(Kd):
            for n in range(N):
                s = 1.0 + sum(float(a[m, c]) * float(dy[m, n]) for m in range(cu[rho], cu[rho + 1]))
                assert wgr[rho, c, n] == np.float32(s)
    assert (fwd[6] == 0).all(), "rows outside every segment are not written"
    assert (wgr[1] == 1).all(), "an empty segment leaves its weight row untouched"


def test_sampled_rows_match_full():
    rng = np.random.default_rng(9)
    G, Kd, N, M = 5, 16, 24, 40
    cu = np.array([0, 7, 7, 20, 33, 40])
    a = synth.to_bf16_bits(rng.standard_normal((M, Kd)).astype(np.float32))
    W = synth.to_bf16_bits(rng.standard_normal((G, Kd, N)).astype(np.float32))
    full = oracle.group_gemm("fwd", a, W, cu, "bf16")
    rows = [0, 6, 7, 19, 39]
    seg, part = oracle.group_gemm_rows("fwd", a, W, cu, rows, "bf16")
    assert seg.tolist() == [0, 0, 2, 2, 4]
    assert (part == full[rows]).all()
    dy = synth.to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    wg = oracle.group_gemm("wgrad", a, dy, cu, "bf16", out=np.zeros((G, Kd, N), np.float32))
    ent = oracle.wgrad_entries(a, dy, cu, 3, [1, 5], [2, 23], "bf16")
    assert np.allclose(ent, [wg[3, 1, 2], wg[3, 5, 23]], rtol=1e-6)


def test_unpermute_reduce_is_the_adjoint_of_the_dispatch():
    """<permute(x), g> summed over every rank's buffer == <x, unpermute_reduce(g)>, float64.

    The dispatch maps each token row to K buffer rows; its adjoint maps a
    buffer gradient back by summing the K rows.  Checked on random real
    values (a property of the definitions, not of the integer fixtures).
    """
    dims = synth.Dims(R=3, S=10, K=3, E=6, B=2, H=5, Hp=4)
    idx, _ = synth.routing(dims, zipf_s=1.0, base_seed=17)
    pl = oracle.plan(idx, dims.E, dims.B)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((dims.R * dims.S, dims.H)).astype(np.float32)
    g = rng.standard_normal((dims.R * dims.SK, dims.H)).astype(np.float32)
    lhs = 0.0
    dest = None
    for q in range(dims.R):
        cu, dest, src = oracle.layout(idx, pl, q)
        xp = oracle.permute(x, src, dims.K, dtype="f32")
        lhs += float(np.sum(xp.astype(np.float64) * g[q * dims.SK:(q + 1) * dims.SK]))
    rhs = 0.0
    for r in range(dims.R):
        # float64 reference of the pulled-back gradient: widen, sum, no rounding
        dx = np.zeros((dims.S, dims.H), np.float64)
        for s_ in range(dims.S):
            for k in range(dims.K):
                d = int(dest[(r * dims.S + s_) * dims.K + k])
                dx[s_] += g[d]
        got = oracle.unpermute_reduce(g, dest, r, dims.S, dims.K, dtype="f32")
        assert (got == dx.astype(np.float32)).all()
        rhs += float(np.sum(x[r * dims.S:(r + 1) * dims.S].astype(np.float64) * dx))
    assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs))


def test_router_weight_grad_is_the_derivative_of_the_combine():
    """Central difference of <dout, combine(w)> in float64 equals combine_weight_grad.

    The combine is linear in each weight, so the difference quotient is exact
    up to float64 rounding; the oracle's float32 result is compared with a
    float32-rounding tolerance.
    """
    dims = synth.Dims(R=2, S=6, K=2, E=4, B=1, H=7, Hp=4)
    idx, w = synth.routing(dims, zipf_s=0.5, base_seed=23)
    pl = oracle.plan(idx, dims.E, dims.B)
    _, dest, _ = oracle.layout(idx, pl, 0)
    rng = np.random.default_rng(4)
    y_all = rng.standard_normal((dims.R * dims.SK, dims.H)).astype(np.float32)
    dout = rng.standard_normal((dims.S, dims.H)).astype(np.float32)
    rank = 1
    got = oracle.combine_weight_grad(y_all, dest, dout, rank, dims.S, dims.K, dtype="f32")

    def loss(wv):
        total = 0.0
        for s_ in range(dims.S):
            row = np.zeros(dims.H, np.float64)
            for k in range(dims.K):
                c = (rank * dims.S + s_) * dims.K + k
                row += wv[c] * y_all[int(dest[c])].astype(np.float64)
            total += float(np.dot(dout[s_].astype(np.float64), row))
        return total

    wf = w.reshape(-1).astype(np.float64)
    for s_ in range(dims.S):
        for k in range(dims.K):
            c = (rank * dims.S + s_) * dims.K + k
            h = 1e-3
            wp, wm = wf.copy(), wf.copy()
            wp[c] += h
            wm[c] -= h
            fd = (loss(wp) - loss(wm)) / (2 * h)
            assert abs(fd - float(got[s_, k])) <= 1e-6 * max(1.0, abs(fd))
