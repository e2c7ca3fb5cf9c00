"""Pins of the gated (SwiGLU) variant of the oracle.

The pages name no activation; the gated unit is the usual framework variant
(READING in the oracle).  Pinned against a library routine (scipy's
logistic function), closed forms of SiLU, central differences of the
forward, and a dense gated MoE written one token copy at a time.
"""
import numpy as np
import pytest
import scipy.special

import oracle
import synth
from oracle.bf16 import bf16_bits_to_f64


def test_silu_is_x_times_the_logistic_function():
    x = np.concatenate([np.linspace(-60, 60, 2001), [-800.0, -40.5, 0.0, 1e-300, 40.5, 800.0]])
    ref = x * scipy.special.expit(x)
    got = oracle.silu(x)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(800.0) == 800.0 and oracle.silu(-800.0) == 0.0


def test_silu_odd_part_is_identity():
    """sigma(x) + sigma(-x) = 1, so silu(x) - silu(-x) = x."""
    x = np.random.default_rng(0).standard_normal(1000) * 7
    assert np.allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=1e-13, atol=1e-13)


def test_backward_matches_central_differences():
    rng = np.random.default_rng(1)
    M, Np = 5, 6
    h = (rng.standard_normal((M, 2 * Np)) * 3).astype(np.float32)
    dz = rng.standard_normal((M, Np)).astype(np.float32)
    got = oracle.swiglu_backward(dz, h, dtype="f32").astype(np.float64)

    def loss(hh):
        z = oracle.silu(hh[:, 0::2]) * hh[:, 1::2]
        return float(np.sum(dz.astype(np.float64) * z))

    h64 = h.astype(np.float64)
    eps = 1e-5
    for i in range(M):
        for j in range(2 * Np):
            hp, hm = h64.copy(), h64.copy()
            hp[i, j] += eps
            hm[i, j] -= eps
            fd = (loss(hp) - loss(hm)) / (2 * eps)
            assert abs(fd - got[i, j]) <= 1e-6 * max(1.0, abs(fd)), (i, j, fd, got[i, j])
    # derivative of silu at 0 is 1/2: with g = 0, u = 1, dz = 1 the gate gradient is 0.5
    d = oracle.swiglu_backward(np.ones((1, 1), np.float32), np.array([[0.0, 1.0]], np.float32),
                               dtype="f32")
    assert d[0, 0] == np.float32(0.5) and d[0, 1] == 0.0


def _dense_gated(x, idx, w, Wu, Wd, dtype):
    """out[t] = round(sum_k w * round(round(silu(x Wg) * (x Wu)) Wd)), pairs interleaved."""
    wid = (lambda a: bf16_bits_to_f64(a)) if dtype == "bf16" else (lambda a: a.astype(np.float64))
    rnd = (lambda a: oracle.f64_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    RS, K = idx.shape[0] * idx.shape[1], idx.shape[2]
    fi, fw = idx.reshape(RS, K), w.reshape(RS, K)
    out = np.zeros((RS, Wd.shape[2]), np.float64)
    for t in range(RS):
        for k in range(K):
            e = fi[t, k]
            xt = wid(x[t])
            gate = xt @ wid(Wu[e])[:, 0::2]
            up = xt @ wid(Wu[e])[:, 1::2]
            z = rnd(gate * scipy.special.expit(gate) * up)
            out[t] += np.float64(fw[t, k]) * wid(rnd(wid(z) @ wid(Wd[e])))
    return rnd(out)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_simulation_matches_dense(dtype):
    dims = synth.Dims(R=3, S=10, K=2, E=6, B=2, H=8, Hp=6)
    idx, w = synth.routing(dims, zipf_s=1.2, base_seed=4)
    pl = oracle.plan(idx, dims.E, dims.B)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((dims.R * dims.S, dims.H)).astype(np.float32)
    Wu = (rng.standard_normal((dims.E, dims.H, 2 * dims.Hp)) * 0.5).astype(np.float32)
    Wd = (rng.standard_normal((dims.E, dims.Hp, dims.H)) * 0.5).astype(np.float32)
    if dtype == "bf16":
        x, Wu, Wd = (synth.to_bf16_bits(a) for a in (x, Wu, Wd))
    Wu_g = np.concatenate([Wu, np.zeros((dims.B,) + Wu.shape[1:], Wu.dtype)])
    Wd_g = np.concatenate([Wd, np.zeros((dims.B,) + Wd.shape[1:], Wd.dtype)])
    Y_all = np.zeros((dims.R * dims.SK, dims.H), x.dtype)
    dest = None
    for q in range(dims.R):
        cu, dest, src = oracle.layout(idx, pl, q)
        xp = oracle.permute(x, src, dims.K, dtype=dtype)
        z, h = oracle.group_gemm_swiglu(xp, oracle.prefetch(Wu_g, pl, q), cu, dtype)
        assert (h == oracle.group_gemm("fwd", xp, oracle.prefetch(Wu_g, pl, q), cu, dtype)).all()
        Y_all[q * dims.SK:(q + 1) * dims.SK] = oracle.group_gemm("fwd", z, oracle.prefetch(Wd_g, pl, q), cu, dtype)
    out = np.concatenate([oracle.combine(Y_all, dest, w, r, dims.S, dims.K, dtype) for r in range(dims.R)])
    ref = _dense_gated(x, idx, w, Wu, Wd, dtype)
    wid = (lambda a: bf16_bits_to_f64(a)) if dtype == "bf16" else (lambda a: a.astype(np.float64))
    # identical operations in a different summation order: equal up to one rounding step
    ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -22
    assert np.allclose(wid(out), wid(ref), rtol=ulp, atol=1e-6)
    assert (out == ref).mean() > 0.9
