"""Host logic of bench.py, on the CPU: it refuses a multi-GPU run before touching a GPU, the
HBM traffic it reports from the committed counter summary goes null as soon as the kernel's
code changes, and the algorithmic bytes and flops behind every roofline fraction are the
sizes of what each kernel must read and write."""
import os
import shutil
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(args, env):
    r = _run_bench(args, env)
    assert r.returncode == 2
    assert "one-GPU share" in r.stderr
    assert r.stdout == ""                       # no JSON line


def test_traffic_only_while_the_kernel_is_unchanged(tmp_path, monkeypatch):
    """recorded_traffic() returns the summary's bytes for a kernel whose source hash is the
    recorded one, keeps them across a comment-only edit, and returns None once the code
    changes."""
    kernel = "gemm_fwd"
    assert bench.recorded_traffic(kernel) is not None, "the committed summary is current"
    src = os.path.join(ROOT, "balanced_token_dispatch_amd", "csrc")
    fake_root = tmp_path / "repo"
    (fake_root / "balanced_token_dispatch_amd").mkdir(parents=True)
    shutil.copytree(src, fake_root / "balanced_token_dispatch_amd" / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    target = fake_root / "balanced_token_dispatch_amd" / "csrc" / "group_gemm.hip"
    text = target.read_text()
    target.write_text(text + "\n// a comment and\n/* a block comment */\n\n")
    assert bench.recorded_traffic(kernel) is not None, "comments do not change the hash"
    target.write_text(text.replace("constexpr int kGroupM = 8;", "constexpr int kGroupM = 4;"))
    assert bench.recorded_traffic(kernel) is None, "a code change invalidates the counters"
    # a kernel with no row in the summary reports none
    assert bench.recorded_traffic("swiglu_bwd") is None


def _shape(R=32, S=4096, K=8, E=256, H=7168, Hp=2048):
    return types.SimpleNamespace(R=R, S=S, K=K, E=E, H=H, Hp=Hp)


def test_algorithmic_work_is_what_each_kernel_moves():
    """Each roofline numerator equals the bytes of the arrays the kernel must touch (or the
    multiply-adds of the products), summed here from array sizes, for the default step."""
    s = _shape()
    SK = s.S * s.K
    bf16, f32, i32 = 2, 4, 4
    work = bench.algorithmic_work(s, n_slots_used=3)
    row = s.H * bf16
    # permute: every received copy's token row read once, its xp row written once, src read
    assert work["permute"] == ("hbm", SK * row + SK * row + SK * i32)
    # weighted permute: the same plus one fp32 weight per copy
    assert work["permute_weighted"] == ("hbm", 2 * SK * row + SK * i32 + SK * f32)
    # combine: each copy's expert row read once, each token's output row written once,
    # dest (int32) and the router weight (fp32) of every copy
    assert work["combine"] == ("hbm", SK * row + s.S * row + SK * (i32 + f32))
    # un-permute reduce: as the combine without the weights
    assert work["unpermute_reduce"] == ("hbm", SK * row + s.S * row + SK * i32)
    # the grouped GEMMs: 2 flops per multiply-add over the rank's SK rows, however the rows
    # split into segments (the figure depends on no routing)
    rng = np.random.default_rng(0)
    cuts = np.sort(rng.integers(0, SK + 1, size=s.E + 7))
    seg = np.diff(np.concatenate([[0], cuts, [SK]]))
    macs = int(sum(int(n) * s.H * s.Hp for n in seg))
    for k in ("gemm_fwd", "gemm_dgrad", "gemm_wgrad", "gemm_fwd_gather", "gemm_wgrad_gather"):
        assert work[k] == ("mfma", 2.0 * macs)
    assert work["gemm_fwd"][1] / 1e9 == pytest.approx(962.07, abs=0.01)
    # fold: per used slot, the home rows read and written and the slot rows read and zeroed
    assert work["fold"] == ("hbm", 3 * 4 * s.H * s.Hp * f32)
    # prefetch: per used slot, the home rows read and the slot rows written
    assert work["prefetch"] == ("hbm", 3 * 2 * s.H * s.Hp * bf16)
    # gated: the up projection twice as wide, so its launches count double in the mean
    g = bench.algorithmic_work(s, n_slots_used=3, gated=True)
    assert g["gemm_fwd_swiglu"][1] == 2 * work["gemm_fwd"][1]
    assert g["gemm_dgrad"][1] == 1.5 * work["gemm_dgrad"][1]


def test_kernel_fracs_from_event_times():
    """kernel_fracs() turns event times into per-launch averages, launches per step and
    fractions of the published peaks (8 TB/s, 2.5 PFLOP/s)."""
    s = _shape()
    SK = s.S * s.K
    fwd_flops = 2.0 * SK * s.H * s.Hp
    permute_bytes = 2.0 * SK * s.H * 2 + 4.0 * SK

    class Timer:
        def ms(self):
            # two steps: two FWD launches per step, one permute per step
            return {"gemm_fwd": [0.8, 0.8, 0.8, 0.8], "permute": [0.2, 0.1]}

    k, totals = bench.kernel_fracs(Timer(), s, n_slots=1, steps=2)
    assert k["gemm_fwd"]["launches_per_step"] == 2
    assert k["gemm_fwd"]["frac"] == pytest.approx(fwd_flops / 0.8e-3 / 2.5e15, abs=1e-4)
    assert k["permute"]["launches_per_step"] == 1
    assert k["permute"]["frac"] == pytest.approx(permute_bytes / 0.15e-3 / 8e12, abs=1e-4)
    assert totals["gemm_fwd"] == pytest.approx(1.6)
    assert totals["permute"] == pytest.approx(0.15)
