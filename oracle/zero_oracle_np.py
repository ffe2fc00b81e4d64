"""Second, independent oracle in NumPy float32 (test infrastructure only).

Written separately from zero_oracle.c so that the two can be checked against
each other bit for bit: NumPy's float32 ufuncs are single IEEE operations with
round-to-nearest-even and no fused multiply-add.  Same readings of the pages as
the C oracle; 16-bit conversions use NumPy's own float16 and a bit-level
bfloat16 definition (the top half of a binary32, rounded to nearest even).
The sum of squares is the correctly rounded fp64 sum (math.fsum), so it may
differ from the C oracle's sequential sum in the last bits only.
"""
import math

import numpy as np

F16, BF16 = 1, 2


def dec(dtype, h):
    h = np.asarray(h, np.uint16)
    if dtype == F16:
        return h.view(np.float16).astype(np.float32)
    return (h.astype(np.uint32) << 16).view(np.float32)


def enc(dtype, x):
    """Round to nearest even into the 16-bit format; every NaN becomes the format's
    positive canonical quiet NaN (0x7E00, 0x7FC0), whatever its sign and payload."""
    x = np.asarray(x, np.float32)
    nan = np.isnan(x)
    if dtype == F16:
        with np.errstate(over="ignore"):
            r = x.astype(np.float16).view(np.uint16).copy()
        r[nan] = 0x7E00
        return r
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def grad_stats(dtype, srcs, inv):
    red = dec(dtype, srcs[0])
    for s in srcs[1:]:
        red = red + dec(dtype, s)
    u = red * np.float32(inv)
    flag = bool((~np.isfinite(u)).any())
    sq = u.astype(np.float64) ** 2
    ss = math.fsum(sq.tolist()) if np.isfinite(sq).all() else float(sq.sum())
    return u, flag, ss


def clip_coef(global_sumsq, max_norm):
    norm = math.sqrt(global_sumsq) if global_sumsq >= 0 else float("nan")
    if not (max_norm > 0):
        return np.float32(1.0), norm
    c = max_norm / (norm + 1e-6)
    return (np.float32(c) if c < 1.0 else np.float32(1.0)), norm


def adam(u, clip, lr, b1, b2, eps, wd, t, w, m, v):
    """One applied step number t (1-based); returns new (w, m, v)."""
    f = np.float32
    b1, b2, lr, eps, wd = f(b1), f(b2), f(lr), f(eps), f(wd)
    p1 = 1.0
    p2 = 1.0
    for _ in range(t):
        p1 *= float(b1)
        p2 *= float(b2)
    bc1, bc2 = f(1.0 - p1), f(1.0 - p2)
    g = u * f(clip)
    m = b1 * m + (f(1.0) - b1) * g
    v = b2 * v + (f(1.0) - b2) * (g * g)
    upd = (m / bc1) / (np.sqrt(v / bc2) + eps)
    w = w - lr * (upd + wd * w)
    return w, m, v
