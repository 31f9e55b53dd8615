"""Pins for the oracle's 8-bit KV cache: the E4M3 codec, the static-scale
quantisation, write_decode_kv_fp8 and paged_gqa_decode_fp8 (CPU only).

The codec is pinned against the format's definition (special values, order,
idempotence), brute-force nearest-value search, and torch's float8_e4m3fn
casts (an independent library implementation of the same OCP format). The
8-bit attention is pinned against the already-pinned bf16 attention: every
E4M3 value is exactly a bf16 value, so a cache of codes must attend exactly
like a bf16 cache holding their decoded values, and the scales must act as
exact multipliers of K and V.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention, bf16, fp8, paged

ALL = np.arange(256, dtype=np.uint8)


def finite_magnitudes():
    return fp8.decode(np.arange(0x7F, dtype=np.uint8))      # codes 0x00 .. 0x7E


# ---------------------------------------------------------------------- codec
def test_decode_all_codes_match_torch_float8_e4m3fn():
    t = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(fp8.decode(ALL), t, equal_nan=True)


def test_decode_special_values():
    d = fp8.decode(ALL)
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    assert d[0x01] == 2.0 ** -9                  # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9              # largest subnormal
    assert d[0x08] == 2.0 ** -6                  # smallest normal
    assert d[0x38] == 1.0                        # exponent field = bias
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.isnan(d).sum() == 2
    assert np.all(np.diff(d[:0x7F]) > 0)         # magnitudes strictly increase
    assert np.array_equal(d[0x80:0xFF], -d[0x00:0x7F])


def test_encode_is_the_inverse_on_every_finite_code():
    d = fp8.decode(ALL)
    fin = ~np.isnan(d)
    assert np.array_equal(fp8.encode(d[fin]), ALL[fin])


def brute_force_encode(x):
    """Nearest finite magnitude by exhaustive search, ties to the even code,
    saturating; sign copied."""
    mags = finite_magnitudes()
    out = []
    for v in np.asarray(x, dtype=np.float64):
        if np.isnan(v):
            out.append(0x7F)
            continue
        a = min(abs(v), 448.0)
        dist = np.abs(mags - a)
        best = np.flatnonzero(dist == dist.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        out.append(c | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8)


def test_encode_matches_brute_force_on_ties_and_random_values():
    mags = finite_magnitudes()
    mids = (mags[:-1] + mags[1:]) / 2                       # exact ties
    rng = np.random.default_rng(7)
    x = np.concatenate([
        mids, -mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
        rng.standard_normal(3000) * 4, rng.standard_normal(500) * 300,
        np.ldexp(rng.uniform(-1, 1, 500), -8),                 # subnormal range
        [0.0, -0.0, 447.9, 448.0, 460.0, 464.0, 470.0, 1e30, -1e30, np.inf, -np.inf, np.nan]])
    assert np.array_equal(fp8.encode(x), brute_force_encode(x))


def test_encode_matches_torch_cast_within_range():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(6),
                        np.float32(finite_magnitudes()[:-1] + np.diff(finite_magnitudes()) / 2)])
    x = np.clip(x, -448, 448).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(x.astype(np.float64)), t)


def test_encode_saturates_and_maps_nan():
    assert list(fp8.encode([449.0, 1e30, np.inf, -500.0, -np.inf, np.nan])) == \
        [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F]


# --------------------------------------------------------------- quantisation
def bf16_values(rng, n, std=1.0):
    return bf16.decode(workloads.bf16_normal(rng, (n,), std))


def test_quantize_with_unit_scale_is_plain_encoding():
    x = bf16_values(np.random.default_rng(9), 5000, 3.0)
    assert np.array_equal(fp8.quantize(x, 1.0), fp8.encode(x))


@pytest.mark.parametrize("k", [-3, -1, 2, 5])
def test_power_of_two_scale_shifts_the_input_exactly(k):
    x = bf16_values(np.random.default_rng(10 + k), 5000, 2.0 ** k)
    assert np.array_equal(fp8.quantize(x, 2.0 ** k), fp8.encode(x * 2.0 ** -k))


@pytest.mark.parametrize("s", [0.37, 1.0, 2.5, 0.0123])
def test_round_trip_error_bound(s):
    """|dequantize(quantize(x)) - x| <= s * half the E4M3 spacing at x / s, plus
    the float32 division's rounding (<= 2^-24 |x|), for |x / s| <= 448."""
    rng = np.random.default_rng(11)
    x = bf16_values(rng, 20000, 100.0 * s)
    x = x[np.abs(x / s) <= 448]
    xs = np.float32(s)
    y = fp8.dequantize(fp8.quantize(x, s), s)
    a = np.abs(x / float(xs))
    e = np.where(a < 2.0 ** -6, -6, np.floor(np.log2(np.maximum(a, 2.0 ** -6))))
    half_spacing = np.ldexp(1.0, (e - 3).astype(np.int64)) / 2
    assert np.all(np.abs(y - x) <= float(xs) * half_spacing * (1 + 2.0 ** -20) + np.abs(x) * 2.0 ** -23)


# --------------------------------------------------- write and attention (fp8)
def fp8_case(cfg, seed, pool="poison"):
    return workloads.make_decode_case(cfg, pool=pool, seed=seed, kv_format="fp8")


def codes_as_bf16_pool(codes):
    """bf16 pool holding the decoded values of E4M3 codes (exact: E4M3 is a
    subset of bf16)."""
    return bf16.encode(fp8.decode(codes))


TINY = workloads.CONFIGS["tiny"]


def test_fp8_attention_equals_bf16_attention_of_the_decoded_cache():
    case = fp8_case(TINY, 21, pool="bench")    # attention alone: the write slot holds a value
    ones = np.ones(TINY.num_kv_heads, np.float32)
    got = attention.paged_gqa_decode_fp8(case.q, case.k_pool, case.v_pool, case.block_table,
                                         case.context_lens, 16, ones, ones)
    ref = attention.paged_gqa_decode(case.q, codes_as_bf16_pool(case.k_pool),
                                     codes_as_bf16_pool(case.v_pool), case.block_table,
                                     case.context_lens, 16)
    assert np.array_equal(got, ref)


def test_fp8_scales_multiply_k_and_v_exactly():
    case = fp8_case(TINY, 22, pool="bench")
    Hkv = TINY.num_kv_heads
    ks = np.array([4.0, 0.5][:Hkv], np.float32)
    vs = np.array([0.25, 2.0][:Hkv], np.float32)
    got = attention.paged_gqa_decode_fp8(case.q, case.k_pool, case.v_pool, case.block_table,
                                         case.context_lens, 16, ks, vs)
    kb = fp8.decode(case.k_pool) * ks[None, :, None, None].astype(np.float64)
    vb = fp8.decode(case.v_pool) * vs[None, :, None, None].astype(np.float64)
    ref = attention.paged_gqa_decode(case.q, bf16.encode(kb), bf16.encode(vb), case.block_table,
                                     case.context_lens, 16)
    assert np.array_equal(got, ref)


def test_fp8_write_touches_exactly_the_new_slots_and_quantises_per_head():
    cfg = workloads.DecodeConfig("w8", batch=3, num_q_heads=8, num_kv_heads=4, head_dim=64,
                                 block_size=16, num_blocks=48, rope_theta=1e4,
                                 ctx_draw="fixed", ctx_fixed=(0, 15, 40), seed=5)
    case = fp8_case(cfg, 23)
    ks = np.array([1.0, 2.0, 0.5, 4.0], np.float32)          # powers of two: exact shifts
    vs = np.array([0.25, 1.0, 8.0, 0.5], np.float32)
    k8, v8, qb, _ = attention.write_decode_kv_fp8(case.k_pool, case.v_pool, case.q, case.k,
                                                  case.v, case.block_table, case.context_lens,
                                                  16, cfg.rope_theta, ks, vs)
    kb, vb, qb2, _ = attention.write_decode_kv(
        np.zeros(case.k_pool.shape, np.uint16), np.zeros(case.v_pool.shape, np.uint16),
        case.q, case.k, case.v, case.block_table, case.context_lens, 16, cfg.rope_theta)
    assert np.array_equal(qb, qb2)
    changed = np.zeros(case.k_pool.shape[:3], bool)
    for b, c in enumerate(case.context_lens):
        blk, off = paged.slot(case.block_table[b], int(c), 16)
        changed[blk, :, off] = True
        for g in range(cfg.num_kv_heads):
            assert np.array_equal(k8[blk, g, off], fp8.encode(bf16.decode(kb[blk, g, off]) / ks[g]))
            assert np.array_equal(v8[blk, g, off], fp8.encode(bf16.decode(case.v[b, g]) / vs[g]))
    assert np.array_equal(k8[~changed], case.k_pool[~changed])
    assert np.array_equal(v8[~changed], case.v_pool[~changed])


def test_fp8_decode_step_nan_poison_never_reaches_the_output():
    case = fp8_case(TINY, 24)
    s = np.array([0.8, 1.3], np.float32)
    out, _, _, _ = attention.decode_step_fp8(case.k_pool, case.v_pool, case.q, case.k, case.v,
                                             case.block_table, case.context_lens, 16,
                                             TINY.rope_theta, s, s)
    assert np.all(np.isfinite(out))


def test_fp8_workload_codes_are_finite_and_normal_like():
    rng = np.random.default_rng(3)
    c = workloads.fp8_normal_like(rng, (200000,))
    d = fp8.decode(c)
    assert np.all(np.isfinite(d))
    assert 0.6 < np.std(d) < 1.4 and abs(np.mean(d)) < 0.02


# ---------------------------------------------------------------- calibration

def _bits(x):
    return bf16.encode(np.asarray(x, dtype=np.float64))


def test_calibrated_scale_maps_each_heads_largest_value_to_448():
    """margin 1: the largest |x| of every head stores as +-448 (code 0x7E or
    0xFE) and nothing saturates; the scale of a head with a negative maximum
    comes from its magnitude."""
    rng = np.random.default_rng(31)
    k = rng.standard_normal((40, 3, 16))
    v = rng.standard_normal((40, 3, 16)) * np.array([1.0, 20.0, 0.01])[None, :, None]
    k[7, 2, 5] = -9.5                                  # head 2's largest magnitude, negative
    kb, vb = _bits(k), _bits(v)
    ks, vs = fp8.calibrate_scales(kb, vb)
    for bits, sc in ((kb, ks), (vb, vs)):
        x = bf16.decode(bits)
        for g in range(3):
            codes = fp8.quantize(x[:, g, :], sc[g])
            mag = codes & 0x7F
            i = np.unravel_index(np.argmax(np.abs(x[:, g, :])), x[:, g, :].shape)
            assert mag[i] == 0x7E
            assert mag.max() == 0x7E and (mag == 0x7E).sum() >= 1
    # per head, not per pool: head 1 of v is 20x head 0 and 2000x head 2
    assert 10 < vs[1] / vs[0] < 40 and 1000 < vs[1] / vs[2] < 4000
    # K and V calibrated separately
    assert not np.array_equal(ks, vs)
    assert np.isclose(ks[2], 9.5 / 448, rtol=1e-6)


def test_calibration_skips_non_finite_values_and_defaults_to_one():
    k = np.zeros((8, 2, 16))
    v = np.ones((8, 2, 16))
    k[:, 1, :] = 0.5
    kb, vb = _bits(k), _bits(v)
    kb[3, 1, 4] = 0x7F80                 # +inf
    kb[4, 1, 4] = 0x7FC0                 # NaN
    vb[:, 0, :] = 0x7F80                 # a head of infinities only
    ks, vs = fp8.calibrate_scales(kb, vb)
    assert ks[0] == np.float32(1.0)      # all zeros
    assert ks[1] == np.float32(np.float32(0.5) / np.float32(448))
    assert vs[0] == np.float32(1.0)      # no finite value
    assert vs[1] == np.float32(np.float32(1.0) / np.float32(448))


def test_calibration_margin_scales_exactly():
    rng = np.random.default_rng(32)
    k = _bits(rng.standard_normal((16, 4, 8)))
    v = _bits(rng.standard_normal((16, 4, 8)))
    k1, v1 = fp8.calibrate_scales(k, v, 1.0)
    k2, v2 = fp8.calibrate_scales(k, v, 2.0)
    np.testing.assert_array_equal(k2, 2 * k1)          # a power of two: exact
    np.testing.assert_array_equal(v2, 2 * v1)
