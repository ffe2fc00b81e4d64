"""The product's 16-bit write-back against the oracle over every float32.

Runs the real step (gradients zero, lr = wd = 0, so every finite master value
is left unchanged by the update) on shards whose fp32 master holds all finite
bit patterns, with the cast fused into the Adam pass and as the standalone
write-back, and compares each 16-bit result with the oracle's encoder.  A
second test does the same for every NaN pattern and +-inf, which the update
turns into NaNs: the write-back must give exactly the canonical quiet NaN."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from zero_partitioned_mixed_reduce_amd.shard import ZeroShard

pytestmark = pytest.mark.gpu
PART = 1 << 30           # patterns per shard


@pytest.fixture(autouse=True)
def _gpu(need_gpu):
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def oracle_encode_parallel(dtype, x):
    n = x.size
    out = np.empty(n, np.uint16)
    step = 1 << 24

    def part(lo):
        out[lo:lo + step] = oracle.encode16(dtype, x[lo:lo + step])

    with ThreadPoolExecutor(16) as ex:
        list(ex.map(part, range(0, n, step)))
    return out


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("fuse", [True, False])
def test_write_back_exhaustive(dtype, fuse):
    bad_total = 0
    for k in range(4):
        print(f"[cast] dtype {dtype} fuse {fuse} patterns {k * PART:#x}..", flush=True)
        bits = torch.arange(k * PART, (k + 1) * PART, dtype=torch.int64, device="cuda").to(torch.int32)
        master = bits.view(torch.float32)
        finite = torch.isfinite(master)
        master = master[finite].contiguous()          # inf and NaN do not survive an update unchanged
        del bits, finite
        n = master.numel()
        params = torch.zeros(n, dtype=torch.int16, device="cuda")
        grads = torch.zeros(n, dtype=torch.int16, device="cuda")
        s = ZeroShard([n], 1, 0, dtype, params, grads=grads, master_init=master)
        s.zero_reduce_grads([], 1.0)
        s.zero_check_overflow(False)
        s.zero_grad_norm(0.0, 0.0)
        s.zero_adam_step(0.0, 0.9, 0.999, 1e-8, 0.0, fuse_cast=fuse)
        if not fuse:
            s.zero_cast_params()
        q = s.query()
        assert not q["skipped"] and q["t"] == 1
        got_w = s.export("master")
        assert torch.equal(got_w.view(torch.int32), master.view(torch.int32))   # the update left w as it was
        x = master.cpu().numpy()
        got = params.cpu().numpy().view(np.uint16)
        s.close()
        del s, master, params, grads, got_w
        torch.cuda.empty_cache()
        exp = oracle_encode_parallel(dtype, x)
        bad = np.flatnonzero(got != exp)
        bad_total += bad.size
        assert bad.size == 0, f"{bad.size} mismatches, first inputs {x[bad[:4]].view(np.uint32)}"
    assert bad_total == 0


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("fuse", [True, False])
def test_write_back_every_nan_and_inf(dtype, fuse):
    """Every float32 NaN pattern (both signs, every payload, quiet and signalling) and
    +-inf as fp32 master values.  The update with lr = wd = 0 turns each into a NaN
    (w - 0 * (upd + 0 * w) is NaN for a NaN or infinite w), and the 16-bit value written,
    fused or standalone, is exactly the write-back's canonical quiet NaN, as the oracle
    encodes it (0x7E00 / 0x7FC0, sign and payload dropped)."""
    print(f"[cast] NaN and inf patterns, dtype {dtype} fuse {fuse}", flush=True)
    payload = torch.arange(1, 1 << 23, dtype=torch.int32, device="cuda")
    neg = torch.tensor(-(1 << 23), dtype=torch.int32, device="cuda")            # 0xFF800000
    bits = torch.cat([payload | 0x7F800000, payload | neg,
                      torch.tensor([0x7F800000], dtype=torch.int32, device="cuda"), neg.view(1)])
    master = bits.view(torch.float32).contiguous()
    n = master.numel()
    assert n == 1 << 24 and int((~torch.isfinite(master)).sum()) == n
    params = torch.zeros(n, dtype=torch.int16, device="cuda")
    grads = torch.zeros(n, dtype=torch.int16, device="cuda")
    s = ZeroShard([n], 1, 0, dtype, params, grads=grads, master_init=master)
    s.zero_reduce_grads([], 1.0)
    s.zero_check_overflow(False)
    s.zero_grad_norm(0.0, 0.0)
    s.zero_adam_step(0.0, 0.9, 0.999, 1e-8, 0.0, fuse_cast=fuse)
    if not fuse:
        s.zero_cast_params()
    q = s.query()
    assert not q["skipped"] and q["t"] == 1
    w_after = s.export("master").cpu().numpy()
    got = params.cpu().numpy().view(np.uint16)
    s.close()
    assert np.isnan(w_after).all()
    exp = oracle_encode_parallel(dtype, w_after)
    canonical = 0x7E00 if dtype == oracle.F16 else 0x7FC0
    assert (exp == canonical).all()
    bad = np.flatnonzero(got != exp)
    assert bad.size == 0, f"{bad.size} mismatches, first written {got[bad[:4]]}"
