"""Pins for the oracle's bf16 codec and paged bookkeeping (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import bf16, paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [list(map(int, ln.split())) for ln in f if ln.strip() and not ln.startswith("#")]


# ------------------------------------------------------------------ bf16 codec
def test_bf16_exhaustive_round_trip():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.decode(bits)
    back = bf16.encode(vals)
    nan = np.isnan(vals)
    assert nan.sum() == 2 * 127           # 0x7F81..0x7FFF and 0xFF81..0xFFFF
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(back[nan] == bf16.QNAN_BITS)


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    d = bf16.decode(bits)
    same = (t == d) | (np.isnan(t) & np.isnan(d))
    assert same.all()


def _all_finite_bf16_sorted():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16.decode(bits)
    keep = np.isfinite(v)
    v, bits = v[keep], bits[keep]
    # drop -0 duplicate of 0 for the search table
    order = np.lexsort((bits, v))
    v, bits = v[order], bits[order]
    uniq = np.concatenate([[True], v[1:] != v[:-1]])
    return v[uniq], bits[uniq]


def test_bf16_encode_is_nearest_brute_force():
    """Nearest-value search over the sorted table of every finite bf16 value,
    ties broken towards the even bit pattern -- an independent method."""
    table, tbits = _all_finite_bf16_sorted()
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-40, 38, 20000),
        rng.uniform(-1e-39, 1e-39, 2000),            # subnormal range
    ])
    x = x[np.abs(x) < 3.3e38]
    enc = bf16.encode(x)
    j = np.searchsorted(table, x)
    lo = table[np.clip(j - 1, 0, len(table) - 1)]
    hi = table[np.clip(j, 0, len(table) - 1)]
    dlo, dhi = np.abs(x - lo), np.abs(x - hi)
    got = bf16.decode(enc)
    best = np.minimum(dlo, dhi)
    assert np.all(np.abs(x - got) == best)


def test_bf16_ties_to_even():
    table, tbits = _all_finite_bf16_sorted()
    pos = (table > 0)
    t, tb = table[pos], tbits[pos]
    mids = (t[:-1] + t[1:]) / 2.0           # exact in float64
    enc = bf16.encode(mids)
    lower_even = (tb[:-1] & 1) == 0
    expect = np.where(lower_even, tb[:-1], tb[1:])
    assert np.array_equal(enc, expect)
    # a hair above / below the midpoint goes to the nearer neighbour
    eps = np.abs(mids) * 2.0 ** -30
    assert np.array_equal(bf16.encode(mids + eps), tb[1:])
    assert np.array_equal(bf16.encode(mids - eps), tb[:-1])


def test_bf16_specials():
    assert bf16.encode(np.array([0.0]))[0] == 0
    assert bf16.encode(np.array([-0.0]))[0] == 0x8000
    assert bf16.encode(np.array([np.inf]))[0] == 0x7F80
    assert bf16.encode(np.array([-np.inf]))[0] == 0xFF80
    assert bf16.encode(np.array([np.nan]))[0] == bf16.QNAN_BITS
    big = (2.0 - 2.0 ** -8) * 2.0 ** 127
    assert bf16.encode(np.array([big]))[0] == 0x7F80
    assert bf16.encode(np.array([np.nextafter(big, 0)]))[0] == 0x7F7F
    assert bf16.encode(np.array([2.0 ** -133]))[0] == 0x0001     # smallest subnormal
    assert bf16.encode(np.array([2.0 ** -134]))[0] == 0x0000     # tie -> even (zero)


def test_bf16_encode_matches_torch_for_float32_inputs():
    rng = np.random.default_rng(1)
    f = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(10000) * 1e-39).astype(np.float32),
        (rng.standard_normal(10000) * 1e38).astype(np.float32),
    ])
    f = f[np.isfinite(f)]
    t = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.encode(f.astype(np.float64)), t)


# ------------------------------------------------------------ paged bookkeeping
def test_block_counts_golden():
    for seq_len, bs, pages in _rows("block_count_pages.txt"):
        assert paged.blocks_needed(seq_len, bs) == pages


def test_block_counts_brute_force():
    for bs in (1, 3, 16, 32):
        for n in range(0, 200):
            count, filled = 0, 0
            for _ in range(n):              # take a page whenever the last is full
                if filled % bs == 0:
                    count += 1
                filled += 1
            assert paged.blocks_needed(n, bs) == count


def test_kv_cache_size_golden():
    (batch, layers, seq, hidden, dt, exact, approx_gb), = _rows("kv_cache_size_inferllm.txt")
    got = paged.kv_cache_bytes(batch, layers, seq, hidden, dt)
    assert got == exact
    assert abs(got / 2 ** 30 - approx_gb) < 0.01


def test_pool_bytes_consistent_with_size_formula():
    # one layer, one "sequence" of N*bs tokens, hidden = Hkv*D: both pools
    N, Hkv, bs, D = 40000, 8, 16, 128
    both = 2 * paged.pool_bytes(N, Hkv, bs, D)
    assert both == paged.kv_cache_bytes(1, 1, N * bs, Hkv * D, 2)
    assert paged.pool_bytes(N, Hkv, bs, D) == 1_310_720_000


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_slot_mapping_equals_append_model(bs):
    rng = np.random.default_rng(bs)
    for ctx in [0, 1, bs - 1, bs, bs + 1, 37, 100, 3 * bs]:
        row = rng.permutation(1000)[: max(1, paged.blocks_needed(ctx, bs))]
        positions, used = paged.append_model_positions(ctx, bs, row)
        assert used == paged.blocks_needed(ctx, bs)
        for p, (blk, off) in enumerate(positions):
            assert paged.slot(row, p, bs) == (blk, off)


def test_element_offset_is_row_major():
    N, Hkv, bs, D = 5, 3, 4, 6
    a = np.arange(N * Hkv * bs * D).reshape(N, Hkv, bs, D)
    for idx in [(0, 0, 0, 0), (4, 2, 3, 5), (2, 1, 0, 3)]:
        assert a[idx] == paged.element_offset(*idx, Hkv, bs, D)


def test_free_stack_lifo_order():
    s = paged.FreeBlockStack(8)
    assert s.alloc(3) == [0, 1, 2]
    assert s.num_free() == 5
    s.free([1, 0])
    assert s.alloc(2) == [0, 1]          # last freed is first handed out
    assert s.alloc(5) == [3, 4, 5, 6, 7]
    assert s.num_free() == 0


def test_free_stack_exhaustion_is_all_or_nothing():
    s = paged.FreeBlockStack(4)
    s.alloc(3)
    with pytest.raises(MemoryError):
        s.alloc(2)
    assert s.num_free() == 1
    assert s.alloc(1) == [3]


def test_free_stack_rejects_double_and_foreign_free():
    s = paged.FreeBlockStack(4)
    ids = s.alloc(2)
    s.free(ids[:1])
    with pytest.raises(ValueError):
        s.free(ids[:1])
    with pytest.raises(ValueError):
        s.free([7])
    with pytest.raises(ValueError):
        s.free([1, 1])
    assert s.num_free() == 3
