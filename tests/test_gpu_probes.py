"""The benchmark's bandwidth probes move the bytes they are credited with: each probe's
output checked on a small ragged size (a partial last block), so the ceilings the
benchmark reports come from kernels that really read and write every element."""
import ctypes

import pytest
import torch

import probes

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(need_gpu):
    yield
    torch.cuda.synchronize()


def st():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("epb,u,bs", [(2048, 2, 256), (2048, 4, 512), (1024, 4, 256), (8192, 1, 256)])
def test_probes_touch_every_element(epb, u, bs):
    n = 3 * epb + 4 * 37                                   # a partial last block
    # finite, normal bf16 bit patterns (0x0080..0x3F7F: 2^-126 <= x < 1), so every sum is a number
    g = torch.randint(0x0080, 0x3F80, (n,), dtype=torch.int16, device="cuda")
    w0, m0, v0 = (torch.randn(n, device="cuda") for _ in range(3))
    w, m, v = w0.clone(), m0.clone(), v0.clone()
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    probes.adam_mix(g.data_ptr(), w.data_ptr(), m.data_ptr(), v.data_ptr(), p.data_ptr(), n, st(), epb, u, bs, 1, 1)
    gf = (g.to(torch.int32) << 16).view(torch.float32)      # the probe's bit move of 16-bit data into fp32
    torch.cuda.synchronize()
    assert torch.equal(w, w0 + gf) and torch.equal(m, m0 + gf) and torch.equal(v, v0 + gf)
    assert torch.equal(p, (w.view(torch.int32) >> 16).to(torch.int16))
    gr = torch.randn(n, device="cuda")
    w2 = w0.clone()
    probes.adam_mix(gr.data_ptr(), w2.data_ptr(), m.data_ptr(), v.data_ptr(), p.data_ptr(), n, st(), epb, u, bs,
                    1, 1, g32=True)
    torch.cuda.synchronize()
    assert torch.equal(w2, w0 + gr)
    dst = torch.zeros(n, device="cuda")
    probes.copy32(w0.data_ptr(), dst.data_ptr(), n, st(), epb, u, bs, 1)
    probes.write32(m.data_ptr(), n, st(), epb, u, bs, 0)
    sink = torch.zeros(n // epb + 1, device="cuda")
    ones = torch.ones(n, device="cuda")
    probes.read32(ones.data_ptr(), n, sink.data_ptr(), st(), epb, u, bs, 1)
    torch.cuda.synchronize()
    assert torch.equal(dst, w0)
    blk = torch.arange(n, device="cuda") // epb
    assert torch.equal(m, blk.to(torch.float32))
    # read32 over ones: a block's first wave leaves 4 x (the quads its 64 lanes visited); lane t of a
    # block of q quads visits quads t, t + bs, t + 2 bs, ... below q
    nb = (n + epb - 1) // epb
    exp_sink = []
    for b in range(nb):
        q = (min(epb, n - b * epb)) // 4
        exp_sink.append(4.0 * sum(max(0, -(-(q - t) // bs)) for t in range(64)))
    assert sink[:nb].cpu().tolist() == exp_sink
    srcs = [torch.randint(0x0080, 0x3F80, (n,), dtype=torch.int16, device="cuda") for _ in range(4)]
    out = torch.zeros(n, device="cuda")
    probes.reduce_mix([x.data_ptr() for x in srcs], out.data_ptr(), n, st(), epb, u, bs, 1)
    torch.cuda.synchronize()
    exp = sum((x.to(torch.int32) << 16).view(torch.float32) for x in srcs)    # the probe's order: ((0 + s0) + s1) + ...
    assert torch.equal(out, exp)
