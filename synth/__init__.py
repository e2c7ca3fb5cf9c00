"""Seeded synthetic inputs for the redundant-expert MoE dispatch path.

This module builds only *inputs*: top-K router outputs (expert ids and
router weights) with a tunable Zipf skew, and dense token / weight /
gradient rows. It holds none of the method's arithmetic (no planning,
no layout, no GEMM, no combine). Both the CPU oracle's tests and the GPU
path's tests and benchmark draw their inputs from here, and from nowhere
else.

Workload recipe (all draws from numpy PCG64 via SeedSequence([base, ...])):

* Router logits for rank p are ``g + b_e`` with ``g ~ N(0, 1)`` float32,
  drawn from the stream SeedSequence([base, p]).  The bias
  ``b_e = -s * ln(1 + rank_pop(e))`` gives expert popularity a Zipf
  shape with exponent ``s`` (s = 0 is unbiased routing).
* ``rank_pop`` places popularity rank i on expert
  ``(R - 1 - i % R) * E_loc + i // R`` ("receiver0": the hottest experts
  are spread one per rank starting from rank R-1, so rank 0 owns the
  coldest expert of each round and ends up hosting replicas), or on
  ``(i % R) * E_loc + i // R`` ("donor0": rank 0 owns the hottest ones).
* Top-K takes the K largest logits, ties to the lower expert id, and
  lists them by (logit descending, id ascending).  Router weights are the
  softmax over the K chosen logits (renormalised top-K softmax), computed
  in float64 and stored as float32.
* Dense rows: tokens and output gradients N(0, 1), expert weights
  N(0, 0.02); bf16 tensors are the float32 draw cast by torch (round to
  nearest even).  Large tensors are drawn on the device with a seeded
  torch generator (see ``device_normal``).

The realised skew of a routing is reported as ``realised_maxvio``, the
statistic that the routing paragraph of the ainovat.com article
"Moonshot AI Open-Sources MoonEP" defines (largest per-expert load over
the perfectly balanced load, minus one).  It is measured here only to
calibrate the Zipf exponent of the generated input.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field, asdict

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
CALIBRATION_FILE = os.path.join(_HERE, "zipf_calibration.json")


@dataclass(frozen=True)
class Dims:
    """Shape of one MoE layer step.

    R ranks, S tokens per rank, K routed experts per token, E experts
    (E_loc = E / R live on each rank), B replica slots per rank, H hidden
    size, Hp expert FFN size (H' on the pages).
    """
    R: int
    S: int
    K: int
    E: int
    B: int
    H: int
    Hp: int

    @property
    def E_loc(self) -> int:
        return self.E // self.R

    @property
    def SK(self) -> int:
        return self.S * self.K

    @property
    def G(self) -> int:
        return self.E + self.B


@dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    dtype: str                      # "f32" or "bf16"
    base_seed: int
    maxvio_targets: tuple           # target skews; None entry = fixed zipf_s
    zipf_s: float | None = None     # fixed exponent (tiny config), else calibrated
    backward: bool = False
    description: str = ""


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", Dims(R=4, S=128, K=2, E=16, B=2, H=256, Hp=512), "f32", 101,
        (None,), zipf_s=1.0,
        description="R4 S128 E16 K2 B2 H256 H'512 fp32, Zipf s=1.0, one projection"),
    "balanced_bf16": Workload(
        "balanced_bf16", Dims(R=8, S=4096, K=6, E=64, B=4, H=2048, Hp=1408), "bf16", 102,
        (None,), zipf_s=0.0,
        description="R8 S4096 E64 K6 B4 H2048 H'1408 bf16, unbiased logits, forward"),
    "skew1_large": Workload(
        "skew1_large", Dims(R=32, S=4096, K=8, E=256, B=8, H=7168, Hp=2048), "bf16", 103,
        (1.0,), description="R32 S4096 E256 K8 B8 H7168 H'2048 bf16, maxvio~1, forward"),
    "skew8_large_fwdbwd": Workload(
        "skew8_large_fwdbwd", Dims(R=32, S=4096, K=8, E=256, B=8, H=7168, Hp=2048), "bf16", 104,
        (8.0,), backward=True,
        description="R32 S4096 E256 K8 B8 H7168 H'2048 bf16, maxvio~8, forward+backward"),
    "sweep_r64": Workload(
        "sweep_r64", Dims(R=64, S=8192, K=8, E=384, B=8, H=7168, Hp=2048), "bf16", 105,
        (0.0, 1.0, 4.0, 16.0), backward=True,
        description="R64 S8192 E384 K8 B8 H7168 H'2048 bf16, maxvio in {0,1,4,16}, fwd+bwd"),
}


# --------------------------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------------------------

def popularity_rank_of_expert(R: int, E: int, placement: str = "receiver0") -> np.ndarray:
    """Inverse of the popularity placement: returns pop[e] = popularity rank of expert e."""
    E_loc = E // R
    i = np.arange(E)
    if placement == "receiver0":
        expert = (R - 1 - (i % R)) * E_loc + i // R
    elif placement == "donor0":
        expert = (i % R) * E_loc + i // R
    else:
        raise ValueError(f"unknown placement {placement!r}")
    pop = np.empty(E, np.int64)
    pop[expert] = i
    return pop


def zipf_bias(R: int, E: int, s: float, placement: str = "receiver0") -> np.ndarray:
    pop = popularity_rank_of_expert(R, E, placement)
    return (-s * np.log1p(pop.astype(np.float64))).astype(np.float32)


def _topk_rows(logits: np.ndarray, K: int):
    """K largest logits per row, ties to the lower column; listed by (value desc, id asc)."""
    S, E = logits.shape
    kth = -np.partition(-logits, K - 1, axis=1)[:, K - 1]
    gt = logits > kth[:, None]
    eq = logits == kth[:, None]
    need = K - gt.sum(axis=1)
    take = gt | (eq & (np.cumsum(eq, axis=1) <= need[:, None]))
    idx = np.nonzero(take)[1].reshape(S, K)            # ascending ids per row
    vals = np.take_along_axis(logits, idx, axis=1)
    order = np.argsort(-vals, axis=1, kind="stable")
    return np.take_along_axis(idx, order, axis=1), np.take_along_axis(vals, order, axis=1)


def routing(dims: Dims, zipf_s: float, base_seed: int, placement: str = "receiver0",
            ranks=None):
    """Top-K router outputs for ranks ``ranks`` (default all R).

    Returns (topk_idx int32 [len(ranks), S, K], topk_w float32 [len(ranks), S, K]).
    Each rank's logits come from its own stream, so any subset of ranks is
    reproducible on its own.
    """
    R, S, K, E = dims.R, dims.S, dims.K, dims.E
    ranks = range(R) if ranks is None else ranks
    bias = zipf_bias(R, E, zipf_s, placement)
    idx_out, w_out = [], []
    for p in ranks:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([base_seed, 1, p])))
        logits = rng.standard_normal((S, E), dtype=np.float32) + bias[None, :]
        idx, vals = _topk_rows(logits, K)
        v = vals.astype(np.float64)
        ex = np.exp(v - v[:, :1])
        w = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
        idx_out.append(idx.astype(np.int32))
        w_out.append(w)
    return np.stack(idx_out), np.stack(w_out)


def balanced_routing(dims: Dims):
    """Exactly balanced routing: copy (p, s, k) goes to expert ((p*S + s)*K + k) mod E.

    Every expert then holds R*S*K/E copies (when E divides R*S*K) and every
    rank's home experts hold exactly S*K copies.  Weights are uniform 1/K.
    """
    R, S, K, E = dims.R, dims.S, dims.K, dims.E
    c = np.arange(R * S * K, dtype=np.int64).reshape(R, S, K)
    idx = (c % E).astype(np.int32)
    w = np.full((R, S, K), 1.0 / K, np.float32)
    return idx, w


def realised_maxvio(topk_idx: np.ndarray, E: int) -> float:
    """Skew of a generated routing: max_e load_e / mean load - 1 (input statistic)."""
    loads = np.bincount(topk_idx.reshape(-1).astype(np.int64), minlength=E)
    return float(loads.max() / (topk_idx.size / E) - 1.0)


def home_load_ratio(topk_idx: np.ndarray, dims: Dims) -> float:
    """Largest per-rank load, over S*K, that static EP with no replicas would see."""
    loads = np.bincount(topk_idx.reshape(-1).astype(np.int64), minlength=dims.E)
    per_rank = loads.reshape(dims.R, dims.E_loc).sum(axis=1)
    return float(per_rank.max() / dims.SK)


def calibrate_zipf(dims: Dims, target: float, base_seed: int, placement="receiver0",
                   tol: float = 0.02, s_hi: float = 4.0, iters: int = 40) -> float:
    """Bisection on the Zipf exponent s, noise fixed, so that realised maxvio ~ target."""
    if target <= 0.0:
        return 0.0

    def mv(s):
        idx, _ = routing(dims, s, base_seed, placement)
        return realised_maxvio(idx, dims.E)

    lo, hi = 0.0, s_hi
    best = None
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        v = mv(mid)
        if best is None or abs(v - target) < abs(best[1] - target):
            best = (mid, v)
        if abs(v - target) <= tol * target:
            return mid
        if v < target:
            lo = mid
        else:
            hi = mid
    return best[0]


def load_calibration() -> dict:
    if not os.path.exists(CALIBRATION_FILE):
        return {}
    with open(CALIBRATION_FILE) as f:
        return json.load(f)


def zipf_for(workload: Workload, target, placement: str = "receiver0") -> float:
    """Zipf exponent for a workload at a target skew (cached calibration, else computed)."""
    if target is None:
        return float(workload.zipf_s)
    if target == 0.0:
        return 0.0
    key = f"{workload.name}:{target:g}:{placement}"
    cal = load_calibration()
    if key in cal:
        return float(cal[key]["zipf_s"])
    return calibrate_zipf(workload.dims, target, workload.base_seed, placement)


# --------------------------------------------------------------------------------------------
# Dense rows
# --------------------------------------------------------------------------------------------

def host_normal(base_seed: int, tag: int, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) array from stream SeedSequence([base, 2, tag])."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([base_seed, 2, tag])))
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def host_ternary(base_seed: int, tag: int, shape, p_zero: float = 0.5) -> np.ndarray:
    """float32 values in {-1, 0, 1}: small integers keep every fp32 partial sum exact."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([base_seed, 3, tag])))
    u = rng.random(shape)
    out = np.where(u < p_zero, 0.0, np.where(u < (1 + p_zero) / 2, 1.0, -1.0))
    return out.astype(np.float32)


def to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """Cast float32 -> bfloat16 with torch (RNE) and return the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def device_normal(shape, std: float, seed: int, dtype, device="cuda", chunk_rows: int = 8192):
    """Seeded N(0, std^2) tensor drawn on the device (for shapes too big to draw on the host).

    The first dimension is drawn in chunks of ``chunk_rows`` from per-chunk
    generators seeded (seed, chunk), so the value of a row does not depend on
    the device's memory size.
    """
    import torch
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    for c0 in range(0, rows, chunk_rows):
        c1 = min(rows, c0 + chunk_rows)
        g = torch.Generator(device=device)
        g.manual_seed((int(seed) * 1000003 + c0 // chunk_rows) & 0x7FFFFFFFFFFFFFFF)
        t = torch.randn((c1 - c0,) + tuple(shape[1:]), generator=g, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out[c0:c1].copy_(t)
    return out


def fill_normal_(t, std: float, seed: int, chunk_rows: int = 8192):
    """Fill a device tensor in place with seeded N(0, std^2) values (chunked over dim 0)."""
    import torch
    rows = t.shape[0]
    flat = t.view(rows, -1)
    for c0 in range(0, rows, chunk_rows):
        c1 = min(rows, c0 + chunk_rows)
        g = torch.Generator(device=t.device)
        g.manual_seed((int(seed) * 1000003 + c0 // chunk_rows) & 0x7FFFFFFFFFFFFFFF)
        r = torch.randn((c1 - c0, flat.shape[1]), generator=g, device=t.device,
                        dtype=torch.float32)
        if std != 1.0:
            r.mul_(std)
        flat[c0:c1].copy_(r)
    return t


__all__ = [
    "Dims", "Workload", "WORKLOADS", "routing", "balanced_routing", "realised_maxvio",
    "home_load_ratio", "calibrate_zipf", "zipf_for", "zipf_bias", "popularity_rank_of_expert",
    "host_normal", "host_ternary", "to_bf16_bits", "device_normal", "fill_normal_",
    "load_calibration",
]
