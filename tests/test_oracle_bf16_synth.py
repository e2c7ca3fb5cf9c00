"""Oracle bf16 rounding vs torch's CPU cast; generator sanity (calibration, shapes, seeds)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.bf16 import f32_to_bf16_bits, bf16_bits_to_f32, f64_to_bf16_bits


def _torch_bits(x32):
    t = torch.from_numpy(x32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_sampled_bit_patterns():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    # ties, near-ties, subnormals, max-finite rounding to inf, zeros, infs
    extra = []
    for hi in (0x0000, 0x0001, 0x3F80, 0x3F81, 0x7F7F, 0x7F7E, 0x8001, 0xBF80, 0xFF7F, 0x0080):
        for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
            extra.append((hi << 16) | lo)
    extra += [0x7F800000, 0xFF800000, 0x00000000, 0x80000000]
    bits = np.concatenate([bits, np.array(extra, np.uint32)])
    x = bits.view(np.float32)
    finite = np.isfinite(x) | np.isinf(x)
    ours = f32_to_bf16_bits(x)
    ref = _torch_bits(x)
    assert (ours[finite] == ref[finite]).all()
    nan = np.isnan(x)
    assert (ours[nan] & 0x7FFF == 0x7FC0).all()
    assert ((ours[nan] & 0x8000) == ((bits[nan] >> 16) & 0x8000)).all()


def test_bf16_widen_is_exact_and_roundtrips():
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(allbits)
    ok = ~np.isnan(f)
    assert (f32_to_bf16_bits(f)[ok] == allbits[ok]).all()
    assert (f64_to_bf16_bits(f.astype(np.float64))[ok] == allbits[ok]).all()


def test_routing_is_deterministic_and_per_rank():
    dims = synth.Dims(R=4, S=32, K=3, E=16, B=2, H=8, Hp=8)
    a, wa = synth.routing(dims, 0.7, 11)
    b, wb = synth.routing(dims, 0.7, 11)
    assert (a == b).all() and (wa == wb).all()
    c, wc = synth.routing(dims, 0.7, 11, ranks=[2])
    assert (c[0] == a[2]).all() and (wc[0] == wa[2]).all()
    assert ((a >= 0) & (a < 16)).all()
    for row in a.reshape(-1, 3):
        assert len(set(row.tolist())) == 3, "top-K picks distinct experts"


def test_topk_tie_rule():
    logits = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], np.float32)
    idx, vals = synth._topk_rows(logits, 2)
    assert idx.tolist() == [[1, 2]]
    idx, vals = synth._topk_rows(logits, 4)
    assert idx.tolist() == [[1, 2, 4, 3]]


def test_zipf_skew_increases_maxvio_and_receiver0_placement():
    dims = synth.Dims(R=8, S=512, K=4, E=32, B=4, H=8, Hp=8)
    mv = [synth.realised_maxvio(synth.routing(dims, s, 5)[0], dims.E) for s in (0.0, 0.5, 1.5)]
    assert mv[0] < mv[1] < mv[2]
    pop = synth.popularity_rank_of_expert(dims.R, dims.E, "receiver0")
    assert sorted(pop.tolist()) == list(range(dims.E))
    # the hottest expert lives on rank R-1, rank 0 owns the coldest of each round
    assert int(np.argmin(pop)) // dims.E_loc == dims.R - 1
    idx, _ = synth.routing(dims, 1.5, 5)
    pl = oracle.plan(idx, dims.E, dims.B)
    assert pl.counts.sum() == idx.size
    assert any(m.rank == 0 for m in pl.replicas), "rank 0 is a receiver"


def test_oracle_maxvio_agrees_with_generator_statistic():
    dims = synth.Dims(R=4, S=100, K=2, E=16, B=2, H=8, Hp=8)
    idx, _ = synth.routing(dims, 1.0, 3)
    pl = oracle.plan(idx, dims.E, dims.B)
    assert oracle.maxvio(pl.T, dims.R, dims.S, dims.K, dims.E) == pytest.approx(
        synth.realised_maxvio(idx, dims.E))


def test_calibration_hits_target_on_small_shape():
    dims = synth.Dims(R=8, S=256, K=4, E=32, B=4, H=8, Hp=8)
    s = synth.calibrate_zipf(dims, 1.0, base_seed=9)
    idx, _ = synth.routing(dims, s, 9)
    assert abs(synth.realised_maxvio(idx, dims.E) - 1.0) <= 0.02


def test_calibration_file_entries_are_consistent():
    cal = synth.load_calibration()
    for key, ent in cal.items():
        name, target, placement = key.split(":")
        assert name in synth.WORKLOADS
        assert abs(ent["maxvio"] - float(target)) <= 0.02 * max(float(target), 1.0)
