"""Host side of the C ABI, on the CPU: the library loads, exports every symbol
the header declares, and its partition and layout agree with the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import zero_partitioned_mixed_reduce_amd as zpm
from zero_partitioned_mixed_reduce_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    """Every function declared in include/*.h."""
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            names |= set(re.findall(r"^\s*(?:zero_status_t|const char\*)\s+(zero_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_header_declares_the_step_calls():
    names = header_functions()
    for required in ("zero_shard_init", "zero_reduce_grads", "zero_check_overflow", "zero_grad_norm",
                     "zero_adam_step", "zero_cast_params", "zero_offload_init", "zero_offload_grad_stats",
                     "zero_offload_adam_step"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    for name in header_functions():
        assert hasattr(L, name), name
        assert name in _abi._PROTOS or name == "zero_last_error"


def test_binding_exposes_same_names():
    for name in header_functions():
        assert hasattr(zpm, name), name


def desc_for(numel, nd, r, dtype=_abi.ZERO_F16, base=1 << 20, per_tensor=False, grads=False, align=0):
    """Description with fake (never dereferenced) 256-byte aligned device addresses."""
    d = _abi.zero_shard_desc_t()
    d.dp_size, d.dp_rank, d.dtype, d.align = nd, r, dtype, align
    arr = (ctypes.c_int64 * len(numel))(*numel)
    d.num_tensors = len(numel)
    d.numel = ctypes.cast(arr, _abi.c_i64p)
    keep = [arr]
    if per_tensor:
        addrs, a = [], base
        for n in numel:
            addrs.append(a)
            a += (2 * n + 255) // 256 * 256 + 256
        p = (ctypes.c_void_p * len(numel))(*addrs)
        keep.append(p)
        d.param16 = ctypes.cast(p, ctypes.POINTER(ctypes.c_void_p))
        if grads:
            g = (ctypes.c_void_p * len(numel))(*[x + (1 << 40) for x in addrs])
            keep.append(g)
            d.grad16 = ctypes.cast(g, ctypes.POINTER(ctypes.c_void_p))
    else:
        d.flat_param16 = base
        if grads:
            d.flat_grad16 = base + (1 << 40)
    d._keep = keep
    return d


CASES = [[1 << 20], [5], [0, 3], [1000, 0, 37, 1], [123457, 99, 640001], [64 * 64 * 3 + 1],
         [4099, (1 << 31) + 12345, 77]]


@pytest.mark.parametrize("numel", CASES)
@pytest.mark.parametrize("nd", [1, 2, 3, 7, 8, 64])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_plan_matches_oracle(numel, nd, per_tensor):
    for r in range(nd):
        info = zpm.zero_shard_plan(desc_for(numel, nd, r, per_tensor=per_tensor))
        psi, S, b, valid = oracle.plan(numel, nd, r)
        assert (info.psi, info.shard_elems, info.shard_begin, info.valid_elems) == (psi, S, b, valid)
        assert info.state_elems >= max(valid, 64) and info.state_elems % 64 == 0
        assert info.model_state_bytes == 4 * psi + 12 * info.state_elems


def test_zero1_7p5b_state_matches_page_formula():
    from oracle.memory import model_state_bytes
    full = zpm.zero_shard_plan(desc_for([7_500_000_000], 64, 0))
    assert abs(full.model_state_bytes - model_state_bytes(1, 7.5e9, 64)) <= 12 * 64
    last = zpm.zero_shard_plan(desc_for([7_500_000_000], 64, 63))
    assert last.valid_elems == 7_500_000_000 - 63 * last.shard_elems
    # the last rank's shard is short by the padding; its state follows its valid length
    assert last.state_elems == (last.valid_elems + 63) // 64 * 64


def test_errors_are_reported():
    d = desc_for([100], 4, 4)
    with pytest.raises(zpm.ZeroError) as e:
        zpm.zero_shard_plan(d)
    assert e.value.status == _abi.ZERO_EINVAL and "dp_rank" in str(e.value)
    d = desc_for([100], 2, 0, dtype=3)
    with pytest.raises(zpm.ZeroError):
        zpm.zero_shard_plan(d)
    d = desc_for([100], 2, 0, align=12)
    with pytest.raises(zpm.ZeroError):
        zpm.zero_shard_plan(d)
    d = desc_for([100, -1], 2, 0)
    with pytest.raises(zpm.ZeroError):
        zpm.zero_shard_plan(d)
    # sizes whose byte counts would leave int64: more than 2^60 elements, more than 2^31 - 1 tensors
    assert zpm.zero_shard_plan(desc_for([1 << 59, 1 << 59], 1 << 30, 0)).psi == 1 << 60   # 2^30-element shard
    for numel in ([1 << 59, 1 << 59, 1], [(1 << 63) - 1, (1 << 63) - 1]):
        with pytest.raises(zpm.ZeroError) as e:
            zpm.zero_shard_plan(desc_for(numel, 1, 0))
        assert e.value.status == _abi.ZERO_EINVAL and "2^60" in str(e.value)
    d = desc_for([100], 1, 0)
    d.num_tensors = 1 << 31                      # numel is never read past the count check
    with pytest.raises(zpm.ZeroError) as e:
        zpm.zero_shard_plan(d)
    assert "num_tensors" in str(e.value)
    # null handles are rejected, not dereferenced
    assert _abi.lib().zero_cast_params(None, None) == _abi.ZERO_EINVAL
    assert "null handle" in zpm.zero_last_error()


def test_abi_from_plain_c(tmp_path):
    """Both headers compile as strict C99 (-Wall -Wextra -pedantic -Werror), and a C program
    linked against the library gets the documented answers from the host-only calls."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib_dir = os.path.dirname(_abi.LIB_PATH)
    exe = tmp_path / "abi_from_c"
    src = os.path.join(ROOT, "tests", "c", "abi_from_c.c")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                        os.path.join(ROOT, "include"), src, "-o", str(exe), "-L", lib_dir, "-lzero_shard",
                        "-Wl,-rpath," + lib_dir], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout and r.stdout.count("ok ") == 12


def test_gpu_c_program_compiles():
    """The plain-C GPU driver of the ABI (tests/c/step_from_c.c) compiles cleanly as C99
    against the headers and the HIP runtime API (it runs in the GPU tests)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if gcc is None or not os.path.isdir(os.path.join(rocm, "include", "hip")):
        pytest.skip("no C compiler or HIP headers")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "step_from_c.c")], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr


def test_static_init_refuses_before_device_work():
    """zero_shard_init_static checks the plan's workspace against the static array
    (ZERO_STATIC_WORKSPACE_BYTES) and the absent caller workspace before any device call,
    so both refusals are visible without a GPU."""
    big = desc_for([2_000_000_000], 1, 0, dtype=_abi.ZERO_BF16)
    info = zpm.zero_shard_plan(big)
    assert info.workspace_bytes > _abi.ZERO_STATIC_WORKSPACE_BYTES
    bufs = _abi.zero_shard_bufs_t()
    bufs.master = bufs.m = bufs.v = 1 << 20                  # never dereferenced: refused first
    bufs.state_capacity = info.state_elems
    h = ctypes.c_void_p()
    assert _abi.lib().zero_shard_init_static(ctypes.byref(big), ctypes.byref(bufs), None, None,
                                             ctypes.byref(h)) == _abi.ZERO_EINVAL
    assert "ZERO_STATIC_WORKSPACE_BYTES" in zpm.zero_last_error() and not h.value
    bufs.workspace = 1 << 21
    small = desc_for([4096], 1, 0, dtype=_abi.ZERO_BF16)
    assert _abi.lib().zero_shard_init_static(ctypes.byref(small), ctypes.byref(bufs), None, None,
                                             ctypes.byref(h)) == _abi.ZERO_EINVAL
    assert "NULL" in zpm.zero_last_error()
    # the header's limit and the binding's agree
    hdr = open(os.path.join(ROOT, "include", "zero_shard.h")).read()
    assert re.search(r"#define ZERO_STATIC_WORKSPACE_BYTES \(8 \* 1024 \* 1024\)", hdr)
    assert _abi.ZERO_STATIC_WORKSPACE_BYTES == 8 * 1024 * 1024


def test_plan_matches_oracle_on_random_lists():
    """Property check over random descriptions (hypothesis): tensor lists of 1-40 tensors
    (empty ones included, totals up to about 2^35 elements), N_d 1-128, every alignment that is a
    multiple of 8 up to 4096, flat or per-tensor parameters.  For every rank the library's plan
    equals the oracle's partition (psi, S, shard start, valid length), the state covers the
    valid elements with at most 7 padding floats per piece plus the 64-float rounding, the
    ranks' valid lengths sum to psi, and the model-state bytes follow 4 psi + 12 state_elems."""
    from hypothesis import given, settings, strategies as st

    @settings(max_examples=150, deadline=None, derandomize=True)
    @given(numel=st.lists(st.one_of(st.just(0), st.integers(1, 70000), st.integers(1, 1 << 30)), min_size=1,
                          max_size=40),
           nd=st.integers(1, 128), align8=st.integers(1, 512), per_tensor=st.booleans(), data=st.data())
    def check(numel, nd, align8, per_tensor, data):
        align = 8 * align8
        ranks = sorted({0, nd - 1, data.draw(st.integers(0, nd - 1))})
        total_valid = 0
        for r in ranks:
            info = zpm.zero_shard_plan(desc_for(numel, nd, r, per_tensor=per_tensor, align=align))
            psi, S, b, valid = oracle.plan(numel, nd, r, align)
            assert (info.psi, info.shard_elems, info.shard_begin, info.valid_elems) == (psi, S, b, valid)
            pieces = oracle.shard_pieces(numel, b, valid)
            assert valid <= info.state_elems <= valid + 8 * len(pieces) + 64
            assert info.model_state_bytes == 4 * psi + 12 * info.state_elems
        for r in range(nd):
            total_valid += oracle.plan(numel, nd, r, align)[3]
        assert total_valid == sum(numel)

    check()
