"""The float64 -> bf16 rounding rule of the RoPE kernels, restated on the CPU.

The write kernels (decode rows, prompt rows, the one-launch step) and the
layer's QKV epilogue round each float64 rotation result once to bf16 through
a float32 rounded to odd, obtained from the hardware's nearest-even
float64 -> float32 conversion: step the nearest value one unit toward zero
when it lies farther from zero than x, set the last bit when inexact, then
round that float32 to bf16 (nearest, ties to even). This test restates the
rule with numpy and checks it against the oracle's bf16 encoder (one exact
rounding straight from float64) on values that reach every case: random
values over the whole exponent range, exact bf16 and float32 values, bf16
ties and values one float64 unit either side of them, float32 subnormals,
the overflow threshold, zeros and NaN.
"""
import numpy as np

from oracle import bf16 as obf16


def rule(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        f = x.astype(np.float32)                       # nearest even
        back = f.astype(np.float64)
    u = f.view(np.uint32).astype(np.uint64)
    inexact = back != x
    away = np.abs(back) > np.abs(x)
    u = np.where(inexact & away, u - 1, u)
    u = np.where(inexact, u | 1, u)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = (u & 0xFFFF).astype(np.uint16)
    out[np.isnan(x)] = obf16.QNAN_BITS
    return out


def _samples():
    rng = np.random.default_rng(11)
    parts = [
        rng.standard_normal(200_000),
        rng.standard_normal(200_000) * np.exp2(rng.integers(-160, 140, 200_000)),
        rng.integers(0, 2 ** 63, 200_000, dtype=np.int64).view(np.float64),
    ]
    # exact bf16 values and the ties halfway between neighbours, and one
    # float64 unit either side of each tie (where a double rounding errs)
    b = rng.integers(0, 0x7F80, 100_000).astype(np.uint16)
    lo = obf16.decode(b)
    hi = obf16.decode(b + 1)
    tie = (lo + hi) / 2
    parts += [lo, -lo, tie, -tie, np.nextafter(tie, np.inf), np.nextafter(tie, -np.inf)]
    f32 = rng.standard_normal(100_000).astype(np.float32).astype(np.float64)
    parts += [f32, f32 * (1 + 2.0 ** -30)]
    parts.append(np.array([0.0, -0.0, np.nan, -np.nan, np.inf, -np.inf,
                           3.3895313892515355e38, 3.3961775292304611e38, 3.39617752923046e38,
                           3.4028234663852886e38, 3.5e38, 1e-39, -1e-39, 1e-45, 2.0 ** -149,
                           2.0 ** -150, 2.0 ** -151, 2.0 ** -133, 2.0 ** -134 * 1.5]))
    x = np.concatenate(parts)
    return x


def test_round_to_odd_rule_is_one_nearest_even_rounding():
    x = _samples()
    got = rule(x)
    want = obf16.encode(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "x=%r rule=%#x exact=%#x" % (x[bad[0]], got[bad[0]], want[bad[0]])


def test_rule_differs_from_two_nearest_roundings():
    """Sanity of the sample: rounding to nearest float32 first and then to bf16
    (the double rounding the rule avoids) does err on some of these values."""
    x = _samples()
    x = x[np.isfinite(x)]
    with np.errstate(over="ignore"):
        u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    twice = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.count_nonzero(twice != obf16.encode(x)) > 0
