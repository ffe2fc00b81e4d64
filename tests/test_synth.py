"""The seeded input generator (CPU side)."""
import numpy as np
import torch

import synth
from synth import recipes


def test_counter_based_slices_agree():
    full = synth.normal_f32(100_000, 7, synth.stream_id(synth.MASTER, 2, 3), 0, 0.02)
    part = synth.normal_f32(1000, 7, synth.stream_id(synth.MASTER, 2, 3), 54_321, 0.02)
    assert (full[54_321:55_321].view(np.uint32) == part.view(np.uint32)).all()
    idx = np.array([0, 5, 99_999, 54_321], np.int64)
    assert (synth.gather_f32(idx, 7, synth.stream_id(synth.MASTER, 2, 3), 0.02) == full[idx]).all()


def test_streams_and_seeds_differ():
    a = synth.normal_f32(1000, 7, 1)
    assert not (a == synth.normal_f32(1000, 7, 2)).any()
    assert not (a == synth.normal_f32(1000, 8, 1)).any()


def test_moments_are_standard_normal_like():
    x = synth.normal_f32(1 << 22, 11, 3).astype(np.float64)
    assert abs(x.mean()) < 3e-3 and abs(x.std() - 1) < 3e-3
    # Irwin-Hall(8) excess kurtosis is -6/(5*8) = -0.15
    k = ((x - x.mean()) ** 4).mean() / x.var() ** 2 - 3
    assert abs(k + 0.15) < 0.02
    assert np.abs(x).max() < 4.9


def test_16bit_values_are_rounded_float_values():
    x = synth.normal_f32(1 << 20, 5, 9, 0, 40.0)
    h = synth.normal_16(1 << 20, synth.F16, 5, 9, 0, 40.0)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert (h == ref).all()
    tiny = synth.normal_f32(1 << 20, 5, 9, 0, 1e-6)      # reaches the fp16 subnormal range
    h = synth.normal_16(1 << 20, synth.F16, 5, 9, 0, 1e-6)
    assert (h == torch.from_numpy(tiny).to(torch.float16).view(torch.int16).numpy().view(np.uint16)).all()
    b = synth.normal_16(1 << 20, synth.BF16, 5, 9, 0, 40.0)
    assert (b == torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)).all()


def test_zero_positions_shared_and_rate():
    n = 1 << 21
    bufs = [synth.normal_16(n, synth.F16, 4, synth.stream_id(synth.GRAD, q), 0, 1e-3, zero_seed=99, zero_mod=1000)
            for q in range(3)]
    z = [b == 0 for b in bufs]
    shared = z[0] & z[1] & z[2]
    assert abs(shared.mean() - 1e-3) < 1e-4
    # a few values also round to zero on their own (|x| < 2^-25); those are not shared
    assert all((zi & ~shared).mean() < 1e-4 for zi in z)


def test_workload_sizes():
    assert recipes.gpt2_shard().psi == 1_555_278_400
    assert recipes.full7p5b().psi == 7_500_000_000
    assert sum(n for _, n in recipes.llama_tensors()) == 6_738_415_616
    assert recipes.tiny().psi == 1 << 20
