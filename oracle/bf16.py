"""bfloat16 codec for the oracle (test infrastructure only).

bfloat16 is the storage type of the K/V cache and of every tensor crossing the
library boundary (the model workloads on the pages run in FP16/BF16: course
project section 2.1, "Qwen3-1.7B (FP16 / BF16)"). bf16 is the upper half of an
IEEE binary32: 1 sign bit, 8 exponent bits, 7 stored significand bits.

* ``decode`` maps bit patterns to float64 exactly.
* ``encode`` rounds a float64 value to the nearest bf16 value, ties to even,
  in ONE rounding straight from float64 (never through float32), with
  overflow to +-inf and NaN to a quiet NaN. This is the definition of
  round-to-nearest-even written out: pick the quantum of the value's binade,
  divide, round half to even, multiply back.
"""
import numpy as np

QNAN_BITS = 0x7FC0

# Largest finite bf16: (2 - 2^-7) * 2^127. Values at or beyond the midpoint to
# 2^128, (2 - 2^-8) * 2^127, round to infinity (the tie goes to the even
# neighbour, and the largest finite value has an odd significand).
_OVERFLOW_MIDPOINT = (2.0 - 2.0 ** -8) * 2.0 ** 127
_EMIN = -126          # smallest normal exponent (shared with binary32)
_MANT_BITS = 7        # stored significand bits


def decode(bits):
    """bf16 bit patterns (uint16 array) -> float64 array, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):        # NaN patterns stay NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def encode(x):
    """float64 array -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    sign = np.signbit(flat_x)
    ax = np.abs(flat_x)

    nan = np.isnan(flat_x)
    inf = (~nan) & (ax >= _OVERFLOW_MIDPOINT)
    zero = ax == 0.0
    fin = ~(nan | inf | zero)

    # exponent of the binade holding |x|, clamped at the subnormal range
    e = np.zeros(ax.shape, dtype=np.int64)
    e[fin] = np.floor(np.log2(ax[fin])).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    lo = np.ldexp(1.0, e)
    too_big = fin & (lo > ax)
    e[too_big] -= 1
    hi = np.ldexp(1.0, e + 1)
    too_small = fin & (hi <= ax)
    e[too_small] += 1
    e = np.maximum(e, _EMIN)

    quantum = np.ldexp(1.0, e - _MANT_BITS)      # spacing of bf16 values in this binade
    scaled = ax / quantum                        # exact: division by a power of two
    rounded = np.rint(scaled)                    # numpy rint rounds half to even
    val = rounded * quantum                      # exact, representable in binary32

    mag = np.zeros(ax.shape, dtype=np.uint16)
    mag[fin] = (val[fin].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    mag[inf] = 0x7F80
    flat_o[:] = mag | (sign.astype(np.uint16) << 15)
    flat_o[nan] = QNAN_BITS
    return out


def round_trip(x):
    """float64 -> nearest bf16 value as float64."""
    return decode(encode(x))
