"""Pins of the oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages print, a closed form,
a library routine, an invariant the pages state, or brute force -- never against
a retyped copy of its own formula alone.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import zero_oracle_np as onp
from oracle.memory import model_state_bytes

F16, BF16 = oracle.F16, oracle.BF16
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def hp_of(lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01):
    return oracle.HParams(lr, b1, b2, eps, wd)


def rand16(dtype, n, sigma, seed):
    r = np.random.default_rng(seed)
    x = (r.standard_normal(n) * sigma).astype(np.float32)
    return oracle.encode16(dtype, x)


# --------------------------------------------------------------------------
# memory accounting printed on the pages


def golden_memory_rows():
    rows = []
    with open(os.path.join(GOLDEN, "memory_totals.txt"), encoding="utf-8") as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            data = line.split("|")[0].split()
            rows.append((int(data[0]), float(data[1]), int(data[2]), int(data[3]), float(data[4]), int(data[5])))
    return rows


@pytest.mark.parametrize("row", golden_memory_rows())
def test_memory_totals_match_pages(row):
    stage, psi, nd, k, printed, dec = row
    gb = model_state_bytes(stage, psi, nd, k) / 1e9
    assert round(gb, dec) == pytest.approx(printed)


def test_memory_exact_values():
    # exact decimal values behind the rounded figures
    assert model_state_bytes(1, 7.5e9, 64) == 31.40625e9
    assert model_state_bytes(2, 7.5e9, 64) == 16.640625e9
    assert model_state_bytes(3, 7.5e9, 64) == 1.875e9


def test_one_gb_model_on_two_gpus():
    # "DeepSpeed ZeRO" ZeRO Stage 1: a 1 GB (fp32) model on 2 GPUs keeps a 500 MB
    # fp16 model on every card, and each card's fp32 optimizer copy of its half is 500 MB.
    psi = 1e9 / 4
    assert 2 * psi == 500e6
    _, S, _, _ = oracle.plan([int(psi)], 2, 0, align=64)
    assert 4 * S == pytest.approx(500e6, abs=4 * 64)


def test_shard_state_matches_stage1_formula():
    # the rank's resident bytes at N_d = 64 for 7.5B: full 16-bit params and grads plus 12 bytes per shard element
    psi = 7_500_000_000
    _, S, _, _ = oracle.plan([psi], 64, 0)
    resident = 2 * psi + 2 * psi + 12 * S
    assert abs(resident - model_state_bytes(1, psi, 64)) <= 12 * 64


# --------------------------------------------------------------------------
# partition


@pytest.mark.parametrize("nd", [1, 2, 3, 4, 7, 8, 64])
@pytest.mark.parametrize("numel", [[1 << 20], [5], [0], [1000, 0, 37, 1], [64 * 64 * 3], [123457, 99, 640001]])
def test_partition_brute_force(nd, numel):
    psi = sum(numel)
    owner = np.full(psi, -1, np.int64)
    shards = []
    for r in range(nd):
        p, S, b, valid = oracle.plan(numel, nd, r)
        assert p == psi
        assert S % 64 == 0 and S * nd >= psi and S * nd - psi < nd * 64 + 64
        assert b == r * S and 0 <= valid <= S
        assert (owner[b:b + valid] == -1).all()
        owner[b:b + valid] = r
        shards.append(S)
    assert (owner >= 0).all()          # union covers [0, psi), disjoint by construction
    assert len(set(shards)) == 1       # equal shard length on every rank


def test_partition_matches_page_formula_when_divisible():
    # "ZeRO 技术原理" 3.3.1: partition_size = tensor_size // world_size; start = partition_size * rank
    for nd in (2, 4, 8, 64):
        size = nd * 64 * 1000
        for r in range(nd):
            _, S, b, valid = oracle.plan([size], nd, r)
            assert S == size // nd and b == (size // nd) * r and valid == S


def test_pieces_cover_shard():
    numel = [100, 3, 0, 77, 1000]
    for nd in (1, 3, 7):
        for r in range(nd):
            _, S, b, valid = oracle.plan(numel, nd, r)
            pieces = oracle.shard_pieces(numel, b, valid)
            assert sum(p[3] for p in pieces) == valid
            off = 0
            starts = np.cumsum([0] + numel)
            for k, toff, soff, ln in pieces:
                assert soff == off and starts[k] + toff == b + soff and 0 <= toff and toff + ln <= numel[k]
                off += ln


# --------------------------------------------------------------------------
# 16-bit formats: exhaustive against library conversions


def _check_encode_chunk(args):
    k, dtype = args
    n = 1 << 24
    x = np.arange(k * n, (k + 1) * n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    got = oracle.encode16(dtype, x)
    tdt = torch.float16 if dtype == F16 else torch.bfloat16
    ref = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    canonical = CANONICAL_NAN[dtype]
    ok = np.where(nan, got == canonical, got == ref)
    return int((~ok).sum())


# The write-back's NaN rule (a reading: the pages are silent): every NaN, of either sign
# and any payload, is written as the format's positive canonical quiet NaN.
CANONICAL_NAN = {F16: 0x7E00, BF16: 0x7FC0}


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_encode_exhaustive_all_float32(dtype):
    """Every one of the 2^32 float32 bit patterns, against torch's CPU conversion
    (round to nearest even, subnormals kept, overflow to infinity) for the non-NaN
    ones, and against the NaN rule (exactly 0x7E00 / 0x7FC0) for the 2^24 - 2 NaN ones."""
    with ThreadPoolExecutor(8) as ex:
        bad = sum(ex.map(_check_encode_chunk, [(k, dtype) for k in range(256)]))
    assert bad == 0


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_nan_rule_every_nan_pattern_both_oracles(dtype):
    """Every float32 NaN pattern (both signs, every payload, quiet and signalling) is
    encoded to the one canonical quiet NaN by the C oracle and by the NumPy mirror;
    +-inf stay +-inf.  A rule that kept the sign or the payload fails here."""
    payload = np.arange(1, 1 << 23, dtype=np.uint32)
    for sign in (0, 1):
        bits = (np.uint32(sign << 31) | np.uint32(0x7F800000) | payload).astype(np.uint32)
        x = bits.view(np.float32)
        assert np.isnan(x).all()
        assert (oracle.encode16(dtype, x) == CANONICAL_NAN[dtype]).all()
        assert (onp.enc(dtype, x) == CANONICAL_NAN[dtype]).all()
    inf = np.array([np.inf, -np.inf], np.float32)
    exp = [0x7C00, 0xFC00] if dtype == F16 else [0x7F80, 0xFF80]
    assert list(oracle.encode16(dtype, inf)) == exp and list(onp.enc(dtype, inf)) == exp
    # the canonical value decodes to a NaN and is a quiet NaN of the format (top fraction bit set)
    assert np.isnan(oracle.decode16(dtype, np.array([CANONICAL_NAN[dtype]], np.uint16)))[0]
    frac_bits = 10 if dtype == F16 else 7
    assert CANONICAL_NAN[dtype] >> (frac_bits - 1) & 1


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_decode_exhaustive(dtype):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode16(dtype, h)
    tdt = torch.float16 if dtype == F16 else torch.bfloat16
    ref = torch.from_numpy(h.view(np.int16)).view(tdt).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan].view(np.uint32) == ref[~nan].view(np.uint32)).all()


def test_round_trip_identity():
    for dtype in (F16, BF16):
        h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        x = oracle.decode16(dtype, h)
        fin = np.isfinite(x)
        assert (oracle.encode16(dtype, x)[fin] == h[fin]).all()


# --------------------------------------------------------------------------
# local reduce, unscale, flag


def test_reduce_exact_on_integer_grid():
    # values k * 2^-10 with |k| <= 1024 are exact in fp16 and bf16-free; any sum of
    # 8 of them is exact in fp32, so the fp32 reduce must equal integer arithmetic.
    nd, n = 8, 5000
    ks = rng.integers(-1024, 1025, size=(nd, n))
    bufs = [oracle.encode16(F16, (k * 2.0 ** -10).astype(np.float32)) for k in ks]
    u, flag, ss = oracle.grad_stats(F16, bufs, 1.0)
    assert not flag
    assert (u.astype(np.float64) == ks.sum(0) * 2.0 ** -10).all()
    # unscale by a power of two is exact
    u2, _, ss2 = oracle.grad_stats(F16, bufs, 1.0 / 1024)
    assert (u2.astype(np.float64) * 1024 == u.astype(np.float64)).all()
    exact = math.fsum(float(v) ** 2 for v in (ks.sum(0) * 2.0 ** -10))
    assert ss == pytest.approx(exact, rel=1e-15)


def test_reduce_is_in_rank_order():
    # fp32 addition is not associative: 1 + 2^-24 + 2^-24 in rank order gives 1,
    # the reverse order gives 1 + 2^-23.  The oracle sums g_0 + g_1 + ... in order.
    a = oracle.encode16(BF16, np.array([1.0], np.float32))
    tiny = oracle.encode16(BF16, np.array([2.0 ** -24], np.float32))
    u, _, _ = oracle.grad_stats(BF16, [a, tiny, tiny], 1.0)
    assert u[0] == np.float32(1.0)
    u, _, _ = oracle.grad_stats(BF16, [tiny, tiny, a], 1.0)
    assert u[0] == np.float32(1.0 + 2.0 ** -23)


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_flag_detects_nonfinite(bad, dtype):
    bufs = [rand16(dtype, 1000, 1e-3, s) for s in range(4)]
    assert not oracle.grad_stats(dtype, bufs, 1.0)[1]
    bufs[2] = bufs[2].copy()
    bufs[2][517] = oracle.encode16(dtype, np.array([bad], np.float32))[0]
    u, flag, _ = oracle.grad_stats(dtype, bufs, 1.0)
    assert flag and not np.isfinite(u[517]) and np.isfinite(np.delete(u, 517)).all()


def test_flag_not_raised_by_large_finite_fp16_sum():
    mx = oracle.encode16(F16, np.array([65504.0], np.float32))
    bufs = [np.repeat(mx, 10) for _ in range(8)]
    u, flag, _ = oracle.grad_stats(F16, bufs, 1.0 / 65536)
    assert not flag and (u == np.float32(8 * 65504.0 / 65536)).all()


# --------------------------------------------------------------------------
# norm and clip


def test_sumsq_against_fsum():
    buf = rand16(F16, 200_000, 3.0, 7)
    u, _, ss = oracle.grad_stats(F16, [buf], 1.0 / 1024)
    exact = math.fsum((u.astype(np.float64) ** 2).tolist())
    assert ss == pytest.approx(exact, rel=1e-12)


def test_norm_constant_vector_closed_form():
    # c * 1_n: norm = |c| sqrt(n); c = 0.5, n = 4^9 gives norm = 256 exactly
    n = 4 ** 9
    buf = oracle.encode16(F16, np.full(n, -0.5, np.float32))
    _, _, ss = oracle.grad_stats(F16, [buf], 1.0)
    clip, norm = oracle.clip_coef(ss, 1.0)
    assert norm == 256.0
    assert clip == np.float32(1.0 / (256.0 + 1e-6))
    clip, _ = oracle.clip_coef(ss, 1000.0)
    assert clip == np.float32(1.0)        # coefficient capped at 1
    clip, _ = oracle.clip_coef(ss, 0.0)
    assert clip == np.float32(1.0)        # max_norm <= 0 disables clipping


@pytest.mark.parametrize("max_norm", [1.0, 0.25, 5.0, 1e4])
def test_clip_coefficient_against_torch(max_norm):
    # torch.nn.utils.clip_grad_norm_ (fp64 on the CPU): coef = max_norm / (total_norm + 1e-6), capped at 1
    g = (rng.standard_normal(4096) * 0.05).astype(np.float32)
    ss = math.fsum((g.astype(np.float64) ** 2).tolist())
    p = torch.nn.Parameter(torch.zeros(4096, dtype=torch.float64))
    p.grad = torch.from_numpy(g.astype(np.float64)).clone()
    total = torch.nn.utils.clip_grad_norm_([p], max_norm, foreach=False)
    coef_t = (p.grad / torch.from_numpy(g.astype(np.float64))).mean().item()
    clip, norm = oracle.clip_coef(ss, max_norm)
    assert norm == pytest.approx(total.item(), rel=1e-14)
    assert clip == pytest.approx(np.float32(min(1.0, coef_t)), rel=2 ** -23)


# --------------------------------------------------------------------------
# Adam


def torch_adamw_steps(w0, grads, lr, b1, b2, eps, wd):
    # the oracle takes every hyperparameter as a binary32 number (and 1 - beta exactly from it);
    # torch gets the same binary32 values
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (lr, b1, b2, eps, wd))
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False, fused=False)
    for g in grads:
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    st = opt.state[p]
    return p.detach().numpy().copy(), st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy()


@pytest.mark.parametrize("wd", [0.0, 0.01, 0.1])
def test_adam_against_torch_adamw(wd):
    """Library routine: torch.optim.AdamW (decoupled weight decay, bias correction)
    on the CPU in fp32; the orders of operations differ, so agreement is to a few
    ulp -- enough to catch a dropped term, a wrong sign or a wrong bias correction."""
    n, steps = 4096, 12
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(steps)]
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    c = oracle.Counters.fresh()
    hp = hp_of(lr, b1, b2, eps, wd)
    for g in grads:
        oracle.adam(False, g, 1.0, hp, c, w, m, v)
    tw, tm, tv = torch_adamw_steps(w0, grads, lr, b1, b2, eps, wd)
    assert c.t == steps
    # tolerances at the scale of the summed terms (|g| ~ 1e-3, |w| ~ 0.02, per-step move ~ lr):
    # cancellation makes relative error near zero meaningless
    np.testing.assert_allclose(m, tm, rtol=0, atol=5e-10)   # ~8 ulp of the largest |m|
    np.testing.assert_allclose(v, tv, rtol=4e-7, atol=1e-16)
    np.testing.assert_allclose(w, tw, rtol=0, atol=6e-8)    # torch rounds (1 - lr wd) to fp32 each step; a wrong decay term is >= 2e-6
    # and a wrong term would be visible: the steps moved w by ~lr per step
    assert np.abs(w - w0).mean() > 0.5 * lr


def test_adam_first_step_closed_form():
    # at t = 1: m = (1-b1) g, v = (1-b2) g^2, mh = g, vh = g^2, so
    # w1 = w0 - lr (g / (|g| + eps) + wd w0) ~= w0 - lr (sign(g) + wd w0)
    n = 2048
    lr, wd, eps = 1e-3, 0.01, 1e-8
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g[:8] = 0.0
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    oracle.adam(False, g, 1.0, hp_of(lr, 0.9, 0.999, eps, wd), oracle.Counters.fresh(), w, m, v)
    f = np.float32
    assert (m == f(1 - f(0.9)) * g).all()
    assert (v == f(1 - f(0.999)) * (g * g)).all()
    g64, w64 = g.astype(np.float64), w0.astype(np.float64)
    expect = w64 - lr * (g64 / (np.abs(g64) + eps) + wd * w64)
    np.testing.assert_allclose(w, expect, rtol=0, atol=4 * np.spacing(np.abs(w0)).max())
    # g = 0: only the decoupled decay acts
    np.testing.assert_allclose(w[:8], w64[:8] * (1 - lr * wd), rtol=2 ** -22)


def test_adam_constant_gradient_bias_correction():
    # with a constant gradient, m_t = g (1-b1^t) and v_t = g^2 (1-b2^t) exactly, so the
    # bias-corrected mh = g and vh = g^2 at every t: each step moves w by lr (g/(|g|+eps) + wd w).
    n, steps = 512, 40
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    w, m, v = np.ones(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    c = oracle.Counters.fresh()
    ref = np.ones(n, np.float64)
    for t in range(1, steps + 1):
        oracle.adam(False, g, 1.0, hp_of(lr, b1, b2, eps, wd), c, w, m, v)
        ref = ref - lr * (g.astype(np.float64) / (np.abs(g.astype(np.float64)) + eps) + wd * ref)
        np.testing.assert_allclose(m / (1 - np.float64(np.float32(b1)) ** t), g, rtol=2e-6)
        np.testing.assert_allclose(v / (1 - np.float64(np.float32(b2)) ** t), g.astype(np.float64) ** 2, rtol=2e-5)
    assert c.t == steps
    assert c.p1 == pytest.approx(float(np.float32(b1)) ** steps, rel=1e-14)
    np.testing.assert_allclose(w, ref, rtol=2e-6)


def test_adam_betas_zero_reduces_to_page_formula():
    # with beta1 = beta2 = 0 and wd = 0 the bias corrections are 1 and the step is the
    # pages' recurrence with m_t = grad, v_t = grad^2: W -= eta * m / (sqrt(v) + eps)
    g = (rng.standard_normal(1000) * 1e-2).astype(np.float32)
    w0 = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    w, m, v = w0.copy(), np.zeros(1000, np.float32), np.zeros(1000, np.float32)
    oracle.adam(False, g, 1.0, hp_of(1e-3, 0.0, 0.0, 1e-8, 0.0), oracle.Counters.fresh(), w, m, v)
    f = np.float32
    assert (m == g).all() and (v == g * g).all()
    assert (w == w0 - f(1e-3) * (g / (np.sqrt(g * g) + f(1e-8)))).all()


def test_gradient_sign_symmetry():
    g = (rng.standard_normal(777) * 1e-2).astype(np.float32)
    outs = []
    for s in (1, -1):
        w, m, v = np.zeros(777, np.float32), np.zeros(777, np.float32), np.zeros(777, np.float32)
        c = oracle.Counters.fresh()
        for _ in range(3):
            oracle.adam(False, s * g, 1.0, hp_of(wd=0.0), c, w, m, v)
        outs.append((w, m, v))
    assert (outs[0][0] == -outs[1][0]).all() and (outs[0][1] == -outs[1][1]).all()
    assert (outs[0][2] == outs[1][2]).all()


# brute force: exact rationals with one explicit binary32 rounding per operation

def f32_round(q: Fraction) -> Fraction:
    """Nearest binary32 value to the rational q, ties to even (subnormals kept)."""
    if q == 0:
        return Fraction(0)
    sgn = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    assert r < Fraction(2) ** 128
    return sgn * r


def f32_sqrt(q: Fraction) -> Fraction:
    """Correctly rounded binary32 square root of a non-negative binary32 value."""
    if q == 0:
        return Fraction(0)
    # scale so the integer square root carries 60+ significant bits, then round with a sticky bit
    k = 200
    num = q.numerator * 4 ** k
    s = math.isqrt(num // q.denominator)
    exact = s * s * q.denominator == num
    approx = Fraction(s, 2 ** k)
    if not exact:
        approx += Fraction(1, 2 ** (k + 1))   # strictly between s and s+1: acts as a sticky bit
    return f32_round(approx)


def F(x):
    return Fraction(float(x))


def brute_adam(u, clip, w, m, v, hp, t):
    b1, b2 = F(np.float32(hp.beta1)), F(np.float32(hp.beta2))
    p1 = p2 = 1.0
    for _ in range(t):
        p1 *= float(np.float32(hp.beta1))
        p2 *= float(np.float32(hp.beta2))
    bc1, bc2 = F(np.float32(1.0 - p1)), F(np.float32(1.0 - p2))
    lr, eps, wd = F(np.float32(hp.lr)), F(np.float32(hp.eps)), F(np.float32(hp.weight_decay))
    omb1, omb2 = f32_round(1 - b1), f32_round(1 - b2)
    R = f32_round
    g = R(u * clip)
    m2 = R(R(b1 * m) + R(omb1 * g))
    v2 = R(R(b2 * v) + R(omb2 * R(g * g)))
    mh, vh = R(m2 / bc1), R(v2 / bc2)
    den = R(f32_sqrt(vh) + eps)
    upd = R(mh / den)
    w2 = R(w - R(lr * R(upd + R(wd * w))))
    return w2, m2, v2


def test_adam_brute_force_exact_rationals():
    n, steps = 24, 4
    hp = hp_of(1e-3, 0.9, 0.999, 1e-8, 0.01)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    W, M, V = [F(x) for x in w], [Fraction(0)] * n, [Fraction(0)] * n
    c = oracle.Counters.fresh()
    for t in range(1, steps + 1):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        g[0] = 0.0
        g[1] = np.float32(1e-30)   # tiny: exercises subnormal squares
        clip = np.float32(0.75)
        oracle.adam(False, g, clip, hp, c, w, m, v)
        for i in range(n):
            W[i], M[i], V[i] = brute_adam(F(g[i]), F(clip), W[i], M[i], V[i], hp, t)
        assert [F(x) for x in w] == W
        assert [F(x) for x in m] == M
        assert [F(x) for x in v] == V


# --------------------------------------------------------------------------
# skip semantics ("DeepSpeed ZeRO", 权重更新的触发条件)


def make_states(dtype, nd, numel, seed):
    states, begins = [], []
    psi = sum(numel)
    master = (np.random.default_rng(seed).standard_normal(psi) * 0.02).astype(np.float32)
    p16_full = oracle.encode16(dtype, master)
    for r in range(nd):
        _, S, b, valid = oracle.plan(numel, nd, r)
        st = oracle.RankState(dtype, p16_full[b:b + valid], master[b:b + valid])
        states.append(st)
        begins.append(b)
    return states, begins, p16_full, master


def snapshot(states):
    return [(s.w.copy(), s.m.copy(), s.v.copy(), s.p16.copy(), s.counters.t, s.counters.p1, s.counters.p2)
            for s in states]


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_skip_leaves_everything_unchanged(bad):
    nd, psi, dtype = 4, 4096 + 17, F16
    states, begins, _, _ = make_states(dtype, nd, [psi], 5)
    hp = hp_of()
    grads = [rand16(dtype, psi, 1.0, 100 + q) for q in range(nd)]
    oracle.step_ranks(states, grads, begins, 1 / 1024, 1.0, hp)           # one applied step
    before = snapshot(states)
    bad_grads = [g.copy() for g in grads]
    bad_grads[0][begins[3] + 7] = oracle.encode16(dtype, np.array([bad], np.float32))[0]  # only in rank 3's shard
    res = oracle.step_ranks(states, bad_grads, begins, 1 / 1024, 1.0, hp)
    assert [r["flag"] for r in res] == [False, False, False, True]
    assert all(r["skipped"] for r in res)
    after = snapshot(states)
    for a, b in zip(before, after):
        for x, y in zip(a, b):
            if isinstance(x, np.ndarray):
                assert (x.view(np.uint8) == y.view(np.uint8)).all()
            else:
                assert x == y


def test_leading_skips_keep_moments_uninitialised():
    # the first 3 steps overflow: moments stay exactly zero and fp16 is not written;
    # the 4th (first good) step equals a fresh first step.
    dtype, psi = F16, 3000
    states, begins, p16_full, master = make_states(dtype, 1, [psi], 9)
    fresh, _, _, _ = make_states(dtype, 1, [psi], 9)
    hp = hp_of()
    good = rand16(dtype, psi, 1.0, 77)
    bad = good.copy()
    bad[5] = 0x7C00
    for _ in range(3):
        res = oracle.step_ranks(states, [bad], begins, 1 / 1024, 1.0, hp)
        assert res[0]["skipped"]
        assert (states[0].m == 0).all() and (states[0].v == 0).all()
        assert (states[0].m.view(np.uint32) == 0).all() and states[0].counters.t == 0
        assert (states[0].p16 == p16_full).all()
    oracle.step_ranks(states, [good], begins, 1 / 1024, 1.0, hp)
    oracle.step_ranks(fresh, [good], begins, 1 / 1024, 1.0, hp)
    assert states[0].counters.t == 1
    for x, y in zip(snapshot(states)[0], snapshot(fresh)[0]):
        if isinstance(x, np.ndarray):
            assert (x.view(np.uint8) == y.view(np.uint8)).all()
        else:
            assert x == y


def test_other_rank_flag_skips():
    states, begins, _, _ = make_states(BF16, 2, [500], 3)
    before = snapshot(states)
    g = rand16(BF16, 500, 1e-3, 4)
    res = oracle.step_ranks(states, [g], begins, 1.0, 1.0, hp_of(), extra_found_inf=True)
    assert all(r["skipped"] for r in res)
    assert all((a[0] == b[0]).all() for a, b in zip(before, snapshot(states)))


# --------------------------------------------------------------------------
# partition invariance ("DeepSpeed ZeRO", ZeRO Stage 2 数学推导)


@pytest.mark.parametrize("nd", [2, 3, 4, 7])
@pytest.mark.parametrize("mode", ["reduce", "flat"])
def test_partition_invariance(nd, mode):
    """The concatenation of the N_d shard updates equals one unpartitioned update,
    bit for bit, given the same global norm (per-parameter independence)."""
    dtype, psi, steps = F16, 10_000 + 37, 3
    hp = hp_of(1e-3, 0.9, 0.999, 1e-8, 0.01)
    states, begins, p16_full, master = make_states(dtype, nd, [psi], 11)
    whole = oracle.RankState(dtype, p16_full, master)
    for s in range(steps):
        if mode == "reduce":
            grads = [rand16(dtype, psi, 300.0, 1000 * s + q) for q in range(nd)]
        else:
            grads = [rand16(dtype, psi, 300.0, 1000 * s)]
        res = oracle.step_ranks(states, grads, begins, 1 / 1024, 1.0, hp)
        clips = {float(r["clip"]) for r in res}
        assert len(clips) == 1 and next(iter(clips)) < 1.0     # the clip is active and identical on all ranks
        u, flag, _ = oracle.grad_stats(dtype, grads, 1 / 1024)
        oracle.adam(flag, u, res[0]["clip"], hp, whole.counters, whole.w, whole.m, whole.v)
        oracle.cast(dtype, whole.w, whole.p16)
    for name in ("w", "m", "v", "p16"):
        cat = np.concatenate([getattr(st, name) for st in states])
        assert (cat.view(np.uint8) == getattr(whole, name).view(np.uint8)).all(), name


def test_global_sum_is_one_rank_order_sum_for_every_rank():
    """Every rank gets the same global sum of squares, the local sums added in rank
    order.  Local sums 1, 2^-53, 2^-53 (bf16 gradients 1.0 on rank 0, two of 2^-27 on
    ranks 1 and 2): in rank order (1 + 2^-53) + 2^-53 rounds to 1 at each addition
    (ties to even), so every rank must see exactly 1.0; a per-rank form ss_r + (sum
    of the others) would give rank 0 1 + 2^-52 and the other ranks 1."""
    nd = 3
    states, begins, _, _ = make_states(BF16, nd, [3 * 64], 5)
    g = np.zeros(3 * 64, np.uint16)
    g[0] = oracle.encode16(BF16, np.array([1.0], np.float32))[0]
    tiny = oracle.encode16(BF16, np.array([2.0 ** -27], np.float32))[0]
    g[begins[1]] = g[begins[1] + 1] = g[begins[2]] = g[begins[2] + 1] = tiny
    res = oracle.step_ranks(states, [g], begins, 1.0, 0.5, hp_of())
    assert [r["local_sumsq"] for r in res] == [1.0, 2.0 ** -53, 2.0 ** -53]
    assert all(r["global_sumsq"] == 1.0 for r in res)
    assert 1.0 + (2.0 ** -53 + 2.0 ** -53) == 1.0 + 2.0 ** -52     # what rank 0's per-rank form would give
    assert all(r["norm"] == 1.0 and r["clip"] == np.float32(0.5 / (1.0 + 1e-6)) for r in res)


# --------------------------------------------------------------------------
# the two oracles agree bit for bit


def test_c_oracle_equals_numpy_oracle_tiny_config():
    """Five steps of the tiny workload (4 ranks, fp16, loss scale 1024, inf in step 2)."""
    nd, psi, dtype = 4, 1 << 16, F16
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    hp = hp_of(lr, b1, b2, eps, wd)
    states, begins, p16_full, master = make_states(dtype, nd, [psi], 21)
    np_w = [st.w.copy() for st in states]
    np_m = [np.zeros_like(st.w) for st in states]
    np_v = [np.zeros_like(st.w) for st in states]
    t_applied = 0
    for s in range(1, 6):
        grads = [rand16(dtype, psi, 1e-3 * 1024, 50 * s + q) for q in range(nd)]
        if s == 2:
            grads[0][3 * begins[1] + 777 if 3 * begins[1] + 777 < psi else 777] = 0x7C00
        res = oracle.step_ranks(states, grads, begins, 1 / 1024, 1.0, hp)
        loc = [onp.grad_stats(dtype, [g[begins[r]:begins[r] + states[r].w.size] for g in grads], 1 / 1024)
               for r in range(nd)]
        flag = any(x[1] for x in loc)
        assert flag == res[0]["skipped"] == (s == 2)
        if flag:
            continue
        t_applied += 1
        clip, _ = onp.clip_coef(math.fsum(x[2] for x in loc), 1.0)
        for r in range(nd):
            assert abs(res[r]["local_sumsq"] - loc[r][2]) <= 1e-12 * loc[r][2]
            assert clip == res[r]["clip"]
            np_w[r], np_m[r], np_v[r] = onp.adam(loc[r][0], clip, lr, b1, b2, eps, wd, t_applied,
                                                 np_w[r], np_m[r], np_v[r])
    for r in range(nd):
        assert (states[r].w.view(np.uint32) == np_w[r].view(np.uint32)).all()
        assert (states[r].m.view(np.uint32) == np_m[r].view(np.uint32)).all()
        assert (states[r].v.view(np.uint32) == np_v[r].view(np.uint32)).all()
        assert (states[r].p16 == onp.enc(dtype, np_w[r])).all()


# --------------------------------------------------------------------------
# gradient accumulation over micro-steps ("DeepSpeed ZeRO", ZeRO Stage 2, 梯度累积)


def test_accumulation_exact_on_integer_grid():
    nd, n, K = 8, 3000, 4
    ks = rng.integers(-256, 257, size=(K, nd, n))
    acc = np.zeros(n, np.float32)
    for k in range(K):
        bufs = [oracle.encode16(F16, (ks[k, q] * 2.0 ** -8).astype(np.float32)) for q in range(nd)]
        oracle.accumulate(F16, bufs, acc, first=(k == 0))
    assert (acc.astype(np.float64) == ks.sum(axis=(0, 1)) * 2.0 ** -8).all()
    u, flag, ss = oracle.stats_f32(acc, 0.25)
    assert not flag and (u.astype(np.float64) == ks.sum(axis=(0, 1)) * 2.0 ** -10).all()


def test_accumulation_adds_the_reduced_micro_step():
    # the micro-step's reduce-scatter result s = g_0 + g_1 is formed first, then added:
    # acc = 1, s = 2^-24 + 2^-24 = 2^-23 gives 1 + 2^-23; adding g_0 then g_1 to acc would give 1
    one = oracle.encode16(BF16, np.array([1.0], np.float32))
    tiny = oracle.encode16(BF16, np.array([2.0 ** -24], np.float32))
    acc = np.zeros(1, np.float32)
    oracle.accumulate(BF16, [one], acc, first=True)
    oracle.accumulate(BF16, [tiny, tiny], acc, first=False)
    assert acc[0] == np.float32(1.0 + 2.0 ** -23)


def test_single_micro_step_equals_plain_intake():
    bufs = [rand16(F16, 5000, 300.0, 40 + q) for q in range(3)]
    acc = np.full(5000, 7.0, np.float32)          # overwritten by the first micro-step
    oracle.accumulate(F16, bufs, acc, first=True)
    u1, f1, s1 = oracle.stats_f32(acc, 1 / 1024)
    u2, f2, s2 = oracle.grad_stats(F16, bufs, 1 / 1024)
    assert (u1.view(np.uint32) == u2.view(np.uint32)).all() and f1 == f2 and s1 == s2


def test_overflow_in_any_micro_step_skips():
    states, begins, _, _ = make_states(F16, 2, [4000], 8)
    before = snapshot(states)
    micro = [[rand16(F16, 4000, 100.0, 60 + k)] for k in range(3)]
    micro[1][0] = micro[1][0].copy()
    micro[1][0][123] = 0x7C00
    res = oracle.step_ranks_accumulated(states, micro, begins, 1 / 1024, 1.0, hp_of())
    assert [r["flag"] for r in res] == [True, False] and all(r["skipped"] for r in res)
    assert all((a[0].view(np.uint32) == b[0].view(np.uint32)).all() for a, b in zip(before, snapshot(states)))


@pytest.mark.parametrize("nd", [2, 5])
def test_partition_invariance_with_accumulation(nd):
    dtype, psi, K = F16, 6001, 3
    hp = hp_of()
    states, begins, p16_full, master = make_states(dtype, nd, [psi], 13)
    whole = oracle.RankState(dtype, p16_full, master)
    micro = [[rand16(dtype, psi, 100.0, 500 + 10 * k + q) for q in range(nd)] for k in range(K)]
    res = oracle.step_ranks_accumulated(states, micro, begins, 1 / 1024, 1.0, hp)
    acc = np.zeros(psi, np.float32)
    for k in range(K):
        oracle.accumulate(dtype, micro[k], acc, first=(k == 0))
    u, flag, _ = oracle.stats_f32(acc, 1 / 1024)
    oracle.adam(flag, u, res[0]["clip"], hp, whole.counters, whole.w, whole.m, whole.v)
    oracle.cast(dtype, whole.w, whole.p16)
    for name in ("w", "m", "v", "p16"):
        cat = np.concatenate([getattr(st, name) for st in states])
        assert (cat.view(np.uint8) == getattr(whole, name).view(np.uint8)).all(), name


# --------------------------------------------------------------------------
# dynamic loss scale ("DeepSpeed ZeRO" 配置说明: loss_scale 0, initial_scale_power 16)


def test_loss_scale_against_torch_amp_update():
    """Library routine: torch's _amp_update_scale_ (the GradScaler state machine) on the CPU."""
    r = np.random.default_rng(99)
    for interval in (1, 3, 7):
        ls = oracle.LossScaler(init_scale=2.0 ** 16, growth=2.0, backoff=0.5, interval=interval, min_scale=2.0 ** -40)
        scale = torch.full((1,), 2.0 ** 16, dtype=torch.float32)
        tracker = torch.zeros(1, dtype=torch.int32)
        for _ in range(200):
            found = bool(r.random() < 0.3)
            ls.update(found)
            torch._amp_update_scale_(scale, tracker, torch.full((1,), float(found)), 2.0, 0.5, interval)
            assert ls.scale.value == scale.item() and ls.good.value == tracker.item()


@pytest.mark.parametrize("interval", [1, 2])
def test_loss_scale_growth_stops_below_infinity_against_torch(interval):
    """From 2^126 with growth 2 the scale reaches 2^127, the largest power of two below
    FLT_MAX, and must stay there: torch's _amp_update_scale_ keeps the old scale when
    scale * growth is not finite.  Also a growth factor of 3 from near FLT_MAX and a
    backoff afterwards (the scale must still come down)."""
    for init, growth in ((2.0 ** 126, 2.0), (1.0e38, 3.0)):
        ls = oracle.LossScaler(init_scale=init, growth=growth, backoff=0.5, interval=interval, min_scale=2.0 ** -40)
        scale = torch.full((1,), init, dtype=torch.float32)
        tracker = torch.zeros(1, dtype=torch.int32)
        for k in range(12):
            found = k == 9
            ls.update(found)
            torch._amp_update_scale_(scale, tracker, torch.full((1,), float(found)), growth, 0.5, interval)
            assert ls.scale.value == scale.item() and ls.good.value == tracker.item(), (init, k)
            assert math.isfinite(ls.scale.value)
        assert ls.scale.value < 3.5e38


def test_loss_scale_closed_forms():
    ls = oracle.LossScaler()                       # 2^initial_scale_power with initial_scale_power = 16
    assert ls.scale.value == 65536.0 and ls.inv == 2.0 ** -16
    for k in range(1, 20):
        ls.update(True)
        assert ls.scale.value == max(2.0 ** (16 - k), 1.0)    # halves down to min_scale and stays
    ls = oracle.LossScaler(init_scale=8.0, interval=4)
    for k in range(1, 13):
        ls.update(False)
        assert ls.scale.value == 8.0 * 2 ** (k // 4) and ls.good.value == k % 4
    ls.update(True)
    assert ls.scale.value == 32.0 and ls.good.value == 0
    assert oracle.LossScaler(init_scale=1000.0).inv == np.float32(1) / np.float32(1000)


# --------------------------------------------------------------------------
# 16-bit output of the local reduce ("DeepSpeed ZeRO", ZeRO Stage 2 基本思想: the fp32
# gradient shard comes from the bf16 reduce-scatter result)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_reduce16_is_the_rounded_fp32_sum(dtype):
    """Against library routines: the rank-order sum in numpy float32, then torch's
    round-to-nearest-even conversion of each sum to the 16-bit type."""
    nd, n = 8, 20_000
    bufs = [rand16(dtype, n, 1.0, 900 + q) for q in range(nd)]
    s = oracle.decode16(dtype, bufs[0]).astype(np.float32)
    for q in range(1, nd):
        s = (s + oracle.decode16(dtype, bufs[q])).astype(np.float32)
    tdt = torch.float16 if dtype == F16 else torch.bfloat16
    exp = torch.from_numpy(s).to(tdt).view(torch.int16).numpy().view(np.uint16)
    assert (oracle.reduce_to16(dtype, bufs) == exp).all()


def test_reduce16_rounds_once_at_the_end():
    # bf16 has 7 fraction bits: 1 + 2^-8 is a tie that rounds to 1.  Rounded once,
    # 1 + 2^-8 + 2^-8 = 1 + 2^-7 is kept; rounding after each addition would give 1.
    one = oracle.encode16(BF16, np.array([1.0], np.float32))
    e = oracle.encode16(BF16, np.array([2.0 ** -8], np.float32))
    assert oracle.decode16(BF16, oracle.reduce_to16(BF16, [one, e, e]))[0] == np.float32(1 + 2.0 ** -7)
    assert oracle.decode16(BF16, oracle.reduce_to16(BF16, [one, e]))[0] == np.float32(1.0)
    # ties go to even: 1 + 2^-7 + 2^-8 -> 1 + 2^-6
    o7 = oracle.encode16(BF16, np.array([1 + 2.0 ** -7], np.float32))
    assert oracle.decode16(BF16, oracle.reduce_to16(BF16, [o7, e]))[0] == np.float32(1 + 2.0 ** -6)


def test_reduce16_exact_grid_and_single_source():
    nd, n = 8, 4000
    ks = rng.integers(-64, 65, size=(nd, n))
    bufs = [oracle.encode16(F16, (k * 2.0 ** -6).astype(np.float32)) for k in ks]
    # |sum| <= 512 on a 2^-6 grid needs at most 16 significant bits -- not exact in fp16 (11),
    # so compare with integer arithmetic rounded by torch; sums below 32 in magnitude are exact
    out = oracle.decode16(F16, oracle.reduce_to16(F16, bufs)).astype(np.float64)
    tot = ks.sum(0) * 2.0 ** -6
    small = np.abs(tot) < 32
    assert (out[small] == tot[small]).all()
    assert (out == torch.tensor(tot, dtype=torch.float64).to(torch.float16).double().numpy()).all()
    one = rand16(BF16, n, 1.0, 77)
    assert (oracle.reduce_to16(BF16, [one]) == one).all()


def test_reduce16_fp16_overflow_skips():
    """Eight ranks of 10000 sum to 80000 > 65504: the fp16 reduce output is +inf, so the
    step is skipped; with the fp32 reduce output the same buffers are finite."""
    big = oracle.encode16(F16, np.array([10000.0], np.float32))
    bufs = [np.repeat(big, 64) for _ in range(8)]
    assert not oracle.grad_stats(F16, bufs, 1.0 / 65536)[1]
    red = oracle.reduce_to16(F16, bufs)
    assert (red == 0x7C00).all() and oracle.grad_stats(F16, [red], 1.0 / 65536)[1]
    states, begins, _, _ = make_states(F16, 2, [64], 31)
    before = snapshot(states)
    res = oracle.step_ranks(states, bufs, begins, 1.0 / 65536, 1.0, hp_of(), reduce_out16=True)
    assert all(r["skipped"] for r in res)
    assert all((a[0].view(np.uint32) == b[0].view(np.uint32)).all() for a, b in zip(before, snapshot(states)))


@pytest.mark.parametrize("nd", [2, 3, 7])
def test_partition_invariance_reduce16(nd):
    dtype, psi, steps = BF16, 9001, 3
    hp = hp_of()
    states, begins, p16_full, master = make_states(dtype, nd, [psi], 41)
    whole = oracle.RankState(dtype, p16_full, master)
    for s in range(steps):
        grads = [rand16(dtype, psi, 0.3, 700 + 10 * s + q) for q in range(nd)]
        res = oracle.step_ranks(states, grads, begins, 1.0, 1.0, hp, reduce_out16=True)
        u, flag, _ = oracle.grad_stats(dtype, [oracle.reduce_to16(dtype, grads)], 1.0)
        oracle.adam(flag, u, res[0]["clip"], hp, whole.counters, whole.w, whole.m, whole.v)
        oracle.cast(dtype, whole.w, whole.p16)
    for name in ("w", "m", "v", "p16"):
        cat = np.concatenate([getattr(st, name) for st in states])
        assert (cat.view(np.uint8) == getattr(whole, name).view(np.uint8)).all(), name


def test_accumulation_of_16bit_reduce_outputs():
    # each micro-step's reduce result is rounded to 16 bits, then added in fp32:
    # micro-step sums 1 + 2^-8 + 2^-8 (kept as 1 + 2^-7) twice accumulate to 2 + 2^-6
    one = oracle.encode16(BF16, np.array([1.0], np.float32))
    e = oracle.encode16(BF16, np.array([2.0 ** -8], np.float32))
    states, begins, _, _ = make_states(BF16, 1, [1], 5)
    micro = [[one, e, e], [one, e, e]]
    acc = np.zeros(1, np.float32)
    for k, srcs in enumerate(micro):
        oracle.accumulate(BF16, [oracle.reduce_to16(BF16, srcs)], acc, first=(k == 0))
    assert acc[0] == np.float32(2 + 2.0 ** -6)
    res = oracle.step_ranks_accumulated(states, micro, begins, 1.0, 0.0, hp_of(), reduce_out16=True)
    assert not res[0]["skipped"] and res[0]["local_sumsq"] == (2 + 2.0 ** -6) ** 2


def test_adam_1000_steps_drift_against_fp64():
    """A sanity bound on accumulated rounding: 1000 oracle steps (fp32, every operation
    rounded) against the same recurrence carried in fp64 from the same fp32
    hyperparameters and gradients.  The fp32 master stays within 1e-5 of the total
    change of the weights, and m and v within 1e-5 of their largest values (measured
    about 1e-6 and below); a wrong bias correction, decay or moment update would be
    off by orders of magnitude more."""
    r = np.random.default_rng(7)
    n = 4096
    w0 = (r.standard_normal(n) * 0.02).astype(np.float32)
    hp = oracle.HParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    ctr = oracle.Counters.fresh()
    W, M, V = w0.astype(np.float64), np.zeros(n), np.zeros(n)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    lr, eps, wd = float(np.float32(1e-3)), float(np.float32(1e-8)), float(np.float32(0.01))
    for t in range(1, 1001):
        g = (r.standard_normal(n) * 1e-3).astype(np.float32)
        oracle.adam(False, g, np.float32(1.0), hp, ctr, w, m, v)
        G = g.astype(np.float64)
        M = b1 * M + (1 - b1) * G
        V = b2 * V + (1 - b2) * G * G
        W = W - lr * ((M / (1 - b1 ** t)) / (np.sqrt(V / (1 - b2 ** t)) + eps) + wd * W)
    assert ctr.t == 1000
    assert np.abs(w - W).max() <= 1e-5 * np.abs(W - w0).max()
    assert np.abs(m - M).max() <= 1e-5 * np.abs(M).max()
    assert np.abs(v - V).max() <= 1e-5 * np.abs(V).max()
