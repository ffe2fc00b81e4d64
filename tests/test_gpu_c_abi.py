"""The step driven from a plain C program through the C ABI on the GPU
(tests/c/step_from_c.c, built by tests/c/build.py and called in-process):
hipMalloc'd buffers, the local reduce of two rank buffers, three steps with an
overflow, checked bit for bit against the C oracle linked into the same
program."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_step_from_c(need_gpu, capfd):
    from tests.c import build as cb
    assert os.path.exists(cb.LIB), "build the C test programs first (__graft_entry__.build())"
    lib = ctypes.CDLL(cb.LIB)
    lib.step_from_c.restype = ctypes.c_int
    print("[c-abi] calling the C program", flush=True)
    rc = lib.step_from_c()
    out = capfd.readouterr().out
    print(out, flush=True)
    assert rc == 0, out
    assert "FAIL" not in out and "ok p16" in out
