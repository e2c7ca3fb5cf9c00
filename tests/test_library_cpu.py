"""libmoe.so loads and exports every symbol include/moe.h declares; host-side checks run
before any HIP call (these tests call no kernel and need no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "balanced_token_dispatch_amd", "libmoe.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def mod():
    if not os.path.exists(LIB):
        pytest.skip("libmoe.so not built")
    import balanced_token_dispatch_amd as m
    return m


def test_header_declares_the_path():
    fns = declared_functions()
    for name in ("moe_plan", "moe_dispatch_layout", "moe_permute", "moe_group_gemm",
                 "moe_combine", "moe_replica_grad_fold", "moe_prefetch", "moe_unpermute_reduce",
                 "moe_combine_weight_grad", "moe_group_gemm_swiglu", "moe_swiglu_backward"):
        assert name in fns


def test_every_declared_symbol_is_exported(mod):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z_]+)$", out, flags=re.M))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    assert set(mod.EXPORTS) == set(declared_functions())


def test_size_queries(mod):
    d = mod.dims(4, 128, 2, 16, 2)
    assert mod.plan_words(d) == 8 + 4 * 16 + 5 * (16 + 4) + 3 * 4 * 2
    assert mod.plan_workspace_bytes(d) > 0
    assert mod.dispatch_layout_workspace_bytes(d) > 0
    for bad in (mod.dims(3, 128, 2, 16, 2),      # E % R != 0
                mod.dims(4, 128, 17, 16, 2),     # K > E
                mod.dims(4, 128, 2, 16, -1),     # B < 0
                mod.dims(0, 128, 2, 16, 2),
                mod.dims(4, 1 << 20, 1024, 1024, 2)):  # R*S*K >= 2^31
        assert mod.plan_words(bad) == 0


def test_host_validation_rejects_before_launch(mod):
    lib = mod.library()
    d = mod.dims(4, 128, 2, 16, 2)
    P = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
    by = ctypes.byref
    assert lib.moe_plan(by(d), None, P, P, None, P, 1 << 20, None) == mod.MOE_EINVAL
    assert lib.moe_plan(by(d), P, P, P, None, P, 1, None) == mod.MOE_ENOSPACE
    bad = mod.dims(3, 128, 2, 16, 2)
    assert lib.moe_plan(by(bad), P, P, P, None, P, 1 << 20, None) == mod.MOE_EINVAL
    assert lib.moe_dispatch_layout(by(d), 4, P, P, P, P, P, P, 1 << 20, None) == mod.MOE_EINVAL
    assert lib.moe_dispatch_layout(by(d), 0, P, P, P, P, P, P, 4, None) == mod.MOE_ENOSPACE
    assert lib.moe_permute(by(d), mod.BF16, 12, P, P, None, P, None) == mod.MOE_EINVAL  # 24 B rows
    assert lib.moe_permute(by(d), 7, 16, P, P, None, P, None) == mod.MOE_EINVAL
    assert lib.moe_combine(by(d), mod.BF16, 16, -1, P, P, P, P, None) == mod.MOE_EINVAL
    assert lib.moe_unpermute_reduce(by(d), mod.BF16, 16, 4, P, P, P, None) == mod.MOE_EINVAL
    assert lib.moe_unpermute_reduce(by(d), mod.BF16, 12, 0, P, P, P, None) == mod.MOE_EINVAL
    assert lib.moe_unpermute_reduce(by(d), mod.F32, 16, 0, None, P, P, None) == mod.MOE_EINVAL
    assert lib.moe_combine_weight_grad(by(d), mod.BF16, 16, -1, P, P, P, P, None) == mod.MOE_EINVAL
    assert lib.moe_combine_weight_grad(by(d), mod.F32, 6, 0, P, P, P, P, None) == mod.MOE_EINVAL
    assert lib.moe_combine_weight_grad(by(d), mod.BF16, 16, 0, P, P, None, P, None) == mod.MOE_EINVAL
    assert lib.moe_replica_grad_fold(by(d), 0, P, P, 6, None) == mod.MOE_EINVAL
    assert lib.moe_prefetch(by(d), 0, P, P, 8, None) == mod.MOE_EINVAL
    gg = lib.moe_group_gemm
    assert gg(mod.GEMM_FWD, mod.BF16, 18, 256, 12, 16, P, P, P, P, None, 0, None) == mod.MOE_EINVAL
    assert gg(mod.GEMM_FWD, mod.BF16, 0, 256, 16, 16, P, P, P, P, None, 0, None) == mod.MOE_EINVAL
    assert gg(5, mod.BF16, 18, 256, 16, 16, P, P, P, P, None, 0, None) == mod.MOE_EINVAL
    assert gg(mod.GEMM_FWD, mod.BF16, 18, 256, 16, 16, None, P, P, P, None, 0, None) == mod.MOE_EINVAL
    # operand tiles are addressed with 32-bit offsets: Kd or N above 2^22 is refused
    assert gg(mod.GEMM_FWD, mod.BF16, 2, 256, (1 << 22) + 8, 16, P, P, P, P, None, 0,
              None) == mod.MOE_EINVAL
    assert gg(mod.GEMM_DGRAD, mod.BF16, 2, 256, 16, (1 << 22) + 8, P, P, P, P, None, 0,
              None) == mod.MOE_EINVAL
    # WGRAD rows are addressed with 32-bit offsets: N above 2^20 is refused
    assert gg(mod.GEMM_WGRAD, mod.BF16, 2, 256, 16, (1 << 20) + 8, P, P, P, P, None, 0,
              None) == mod.MOE_EINVAL
    need = mod.group_gemm_workspace_bytes(mod.GEMM_FWD)
    assert need > 0 and mod.group_gemm_workspace_bytes(mod.GEMM_WGRAD) == 0
    assert mod.group_gemm_workspace_bytes(mod.GEMM_FWD, mod.F32) == 0
    assert gg(mod.GEMM_FWD, mod.BF16, 18, 256, 16, 16, P, P, P, P, P, need - 1, None) == mod.MOE_ENOSPACE
    assert gg(mod.GEMM_DGRAD, mod.BF16, 18, 256, 16, 16, P, P, P, P, P, 0, None) == mod.MOE_ENOSPACE
    sw = lib.moe_group_gemm_swiglu
    assert sw(mod.BF16, 18, 256, 16, 24, P, P, P, P, None, None, 0, None) == mod.MOE_EINVAL  # N%16
    assert sw(mod.F32, 18, 256, 16, 32, P, P, P, P, None, None, 0, None) == mod.MOE_EINVAL   # bf16
    assert sw(mod.BF16, 18, 256, 16, 32, P, P, P, None, None, None, 0, None) == mod.MOE_EINVAL
    assert sw(mod.BF16, 18, 256, 16, 32, P, P, P, P, None, P, need - 1, None) == mod.MOE_ENOSPACE
    assert lib.moe_swiglu_backward(mod.BF16, 4, 4, P, P, P, None) == mod.MOE_EINVAL  # 8 B rows
    assert lib.moe_swiglu_backward(mod.F32, 4, 8, None, P, P, None) == mod.MOE_EINVAL
    assert lib.moe_status_string(mod.MOE_ENOSPACE).startswith(b"workspace")


def test_group_gemm_gather_host_checks(mod):
    """moe_group_gemm_gather refuses DGRAD, fp32, an empty source, a zero divisor, null
    pointers and a short workspace before anything is launched."""
    lib = mod.library()
    P = ctypes.c_void_p(16)  # never dereferenced
    gg = lib.moe_group_gemm_gather
    ok = (mod.GEMM_FWD, mod.BF16, 18, 256, 64, 64, P, 100, P, 2, P, P, P, None, 0, None)
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return gg(*a)
    assert call(a0=mod.GEMM_DGRAD) == mod.MOE_EINVAL
    assert call(a1=mod.F32) == mod.MOE_EINVAL
    assert call(a7=0) == mod.MOE_EINVAL           # no source rows
    assert call(a7=1 << 31) == mod.MOE_EINVAL     # source rows >= 2^31
    assert call(a9=0) == mod.MOE_EINVAL           # gather divisor
    assert call(a6=None) == mod.MOE_EINVAL
    assert call(a8=None) == mod.MOE_EINVAL
    assert call(a4=12) == mod.MOE_EINVAL          # Kd % 8
    assert call(a2=0) == mod.MOE_EINVAL
    need = mod.group_gemm_workspace_bytes(mod.GEMM_FWD)
    assert call(a13=P, a14=need - 1) == mod.MOE_ENOSPACE
    assert call(a0=mod.GEMM_WGRAD, a5=(1 << 20) + 8) == mod.MOE_EINVAL


def test_plan_noalloc_host_checks(mod):
    """moe_plan_noalloc: bad arguments and plans whose scratch exceeds the static array are
    refused before anything touches the GPU; the binding's size constant is the header's."""
    text = open(HEADER).read()
    m = re.search(r"#define MOE_PLAN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mod.PLAN_NOALLOC_SCRATCH_BYTES
    lib = mod.library()
    P = ctypes.c_void_p(16)  # never dereferenced
    by = ctypes.byref
    d = mod.dims(4, 128, 2, 16, 2)
    assert lib.moe_plan_noalloc(by(d), None, P, P, None, None) == mod.MOE_EINVAL
    assert lib.moe_plan_noalloc(by(d), P, None, P, None, None) == mod.MOE_EINVAL
    assert lib.moe_plan_noalloc(by(mod.dims(3, 128, 2, 16, 2)), P, P, P, None, None) == mod.MOE_EINVAL
    for ok in (mod.dims(32, 4096, 8, 256, 8), mod.dims(64, 8192, 8, 384, 8)):
        assert mod.plan_workspace_bytes(ok) <= mod.PLAN_NOALLOC_SCRATCH_BYTES
    big = mod.dims(512, 8192, 8, 1024, 8)
    assert mod.plan_workspace_bytes(big) > mod.PLAN_NOALLOC_SCRATCH_BYTES
    assert lib.moe_plan_noalloc(by(big), P, P, P, None, None) == mod.MOE_ENOSPACE


def test_oracle_is_not_reachable_from_the_product():
    """The binding and the kernels never import or name the oracle."""
    pkg = os.path.join(ROOT, "balanced_token_dispatch_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src, f
