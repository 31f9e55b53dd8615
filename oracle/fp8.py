"""8-bit KV cache: E4M3 codec and per-head static-scale quantisation
(test infrastructure only).

Pages followed:

* vLLM-based inference-framework project report (gitlink.org.cn), the
  technical exploration "FP8 KV Cache quantisation": the KV cache is stored
  in FP8 instead of FP16, which cuts the bytes the attention moves; it was
  measured with vLLM's FP8 KV cache. The report gives no format details, so
  the FP8 KV cache of that engine is read in: E4M3 codes, and one static
  scale per key cache and per value cache (a stored value is x / scale,
  dequantised as code * scale). The scale is kept per KV head here (a single
  per-layer scale is the special case of equal entries), following the
  nxmr.cn inference-techniques article, section 2.2, which reports that
  heads with different value ranges need their own quantisation.
* The same article's section 2.2 also sketches a symmetric int8 scheme with
  scale 127 / max|x| over 64-token groups. Its scale needs the maximum of a
  whole group, which a one-token decode append does not have until the group
  is complete; that scheme is not the one modelled here.

E4M3 (the "FN" variant of the OCP 8-bit floating-point specification): 1
sign bit, 4 exponent bits with bias 7, 3 stored significand bits; exponent
field 0 holds the subnormals m * 2^-9; exponent 15 with significand 7 is NaN;
there are no infinities; the largest finite magnitude is 448.

* ``decode``: code -> float64, exactly.
* ``encode``: float32/float64 value -> code, round to nearest, ties to the
  even code, saturating: magnitudes beyond 448 store +-448. NaN stores 0x7F.
  Written as the definition of rounding: the quantum of the value's binade
  (2^(e - 3) for normals, 2^-9 below 2^-6), divide, round half to even,
  multiply back.
* ``quantize``: the stored code of a bf16 value x under scale s is
  encode(float32(float32(x) / float32(s))) -- the division is one IEEE
  float32 operation (the precision the device computes it in), then a
  single rounding to E4M3.
* ``dequantize``: decode(code) * s in float64 (exact).
* ``calibrate_scales``: static per-head scales from sample rows of k and v
  (for example a prefill chunk). The article's section 2.2 scales a group by
  its largest magnitude (127 / max|x| for int8): the largest value maps to
  the largest code. For E4M3 that reads s = max|x| / 448, here with a
  caller's margin factor (a margin above 1 leaves room for later values
  above the sample's maximum, which would otherwise saturate).
"""
import numpy as np

NAN_CODE = 0x7F
MAX_FINITE = 448.0
_EMIN = -6          # exponent of the smallest normal, 2^-6
_MANT_BITS = 3


def decode(codes):
    """E4M3 codes (uint8 array) -> float64 array, exactly."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m.astype(np.float64), -9)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def encode(x):
    """Values -> E4M3 codes (uint8): nearest, ties to even, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    nan = np.isnan(flat)
    sign = np.signbit(flat)
    ax = np.minimum(np.abs(np.where(nan, 0.0, flat)), MAX_FINITE)

    e = np.full(ax.shape, _EMIN, dtype=np.int64)
    big = ax >= 2.0 ** _EMIN
    e[big] = np.floor(np.log2(ax[big])).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    e[big & (np.ldexp(1.0, e) > ax)] -= 1
    e[big & (np.ldexp(1.0, e + 1) <= ax)] += 1
    quantum = np.ldexp(1.0, e - _MANT_BITS)
    k = np.rint(ax / quantum)                  # ties to even (exact: a power-of-two quotient)
    mag = k * quantum                          # nearest representable magnitude
    # rebuild the code of mag: subnormal field, or exponent / significand
    code = np.empty(ax.shape, dtype=np.int64)
    sub = mag < 2.0 ** _EMIN
    code[sub] = np.rint(mag[sub] / 2.0 ** -9).astype(np.int64)
    ns = ~sub
    if ns.any():
        en = np.floor(np.log2(mag[ns])).astype(np.int64)
        en[np.ldexp(1.0, en) > mag[ns]] -= 1
        mn = np.rint((mag[ns] / np.ldexp(1.0, en) - 1.0) * 8.0).astype(np.int64)
        code[ns] = ((en + 7) << 3) | mn
    code = code | np.where(sign, 0x80, 0)
    code[nan] = NAN_CODE
    out[:] = code.astype(np.uint8)
    return out.reshape(x.shape)


def quantize(bf16_values, scale):
    """Stored codes of bf16 values (as float64 here, exactly representable)
    under one scale: encode(float32(x) / float32(scale)) with the division a
    single float32 operation."""
    xf = np.asarray(bf16_values, dtype=np.float64).astype(np.float32)
    q = xf / np.float32(scale)
    return encode(q.astype(np.float64))


def dequantize(codes, scale):
    """Values an attention reads back: decode(code) * scale (float64, exact)."""
    return decode(codes) * float(np.float32(scale))


def calibrate_scales(k_bits, v_bits, margin=1.0):
    """Per-KV-head scales from sample rows: k_bits, v_bits are bf16 bit
    patterns [rows, num_kv_heads, head_dim]. For each head and each of K and
    V, a = the largest |x| over the head's finite values; the scale is
    float32(float32(a * margin) / 448) (two float32 operations, the precision
    the device computes in), or 1.0 when that is not a positive finite value
    (no finite nonzero sample). Returns (k_scales, v_scales), float32 arrays
    [num_kv_heads]."""
    m = np.float32(margin)

    def per_head(bits):
        b = np.asarray(bits, dtype=np.uint16)
        x = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        hkv = x.shape[1]
        out = np.empty(hkv, dtype=np.float32)
        for g in range(hkv):
            vals = x[:, g, :]
            fin = vals[np.isfinite(vals)]
            a = np.float32(np.max(np.abs(fin))) if fin.size else np.float32(0.0)
            with np.errstate(over="ignore"):
                s = np.float32(np.float32(a * m) / np.float32(MAX_FINITE))
            out[g] = s if (np.isfinite(s) and s > 0) else np.float32(1.0)
        return out

    return per_head(k_bits), per_head(v_bits)
