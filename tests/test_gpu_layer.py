"""GPU parity of the full decoder-layer decode step against the fp64 oracle,
through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_246_amd as mk
import workloads
from oracle import bf16 as obf16
from oracle import layer as olayer
from oracle import rope as orope
from tests.gpu_harness import DEV, bits_to_dev, check_tolerance, dev_to_bits

pytestmark = pytest.mark.gpu

SMALL = workloads.DecodeConfig(
    "small_layer", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
    num_blocks=64, rope_theta=1e4, ctx_draw="fixed", ctx_fixed=(0, 20, 47), seed=11,
    hidden=256, intermediate=512, rms_eps=1e-6)

WIDE = workloads.DecodeConfig(
    "wide_layer", batch=20, num_q_heads=4, num_kv_heads=4, head_dim=128, block_size=16,
    num_blocks=512, rope_theta=1e6, ctx_draw="uniform", ctx_lo=0, ctx_hi=200, seed=12,
    hidden=512, intermediate=768, rms_eps=1e-5)


# The largest batch (32: two 16-row MFMA tiles), an 8-head query group and a
# 3x hidden intermediate: every projection's workgroup runs more epilogue
# items than it has threads. Tested with weights N(0, 0.02), as in the
# Qwen3-8B-shaped workload, and N(0, 0.05), where the outputs reach |20|:
# there a bf16 rounding of the rotated query or of the attention output would
# alone move the result past the elementwise bound, so the layer keeps both
# at about 16 significant bits (bf16 pairs, float32).
MAXB = workloads.DecodeConfig(
    "max_batch_layer", batch=32, num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=16,
    num_blocks=1024, rope_theta=1e6, ctx_draw="uniform", ctx_lo=0, ctx_hi=300, seed=13,
    hidden=1024, intermediate=3072, rms_eps=1e-6)


# Batch 12: one 16-row tile with more than 8 rows (the projections' two-load
# fp32 activation form); batch 1: the one-load form with a single valid row.
MID = workloads.DecodeConfig(
    "mid_batch_layer", batch=12, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
    num_blocks=256, rope_theta=1e6, ctx_draw="uniform", ctx_lo=0, ctx_hi=150, seed=14,
    hidden=768, intermediate=1536, rms_eps=1e-6)
# Batch 17: the second 16-row tile holds one row.
B17 = workloads.DecodeConfig(
    "b17_layer", batch=17, num_q_heads=8, num_kv_heads=4, head_dim=64, block_size=16,
    num_blocks=256, rope_theta=1e4, ctx_draw="uniform", ctx_lo=0, ctx_hi=120, seed=16,
    hidden=512, intermediate=768, rms_eps=1e-6)
ONE = workloads.DecodeConfig(
    "one_row_layer", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=16,
    num_blocks=32, rope_theta=1e4, ctx_draw="fixed", ctx_fixed=(33,), seed=15,
    hidden=512, intermediate=1024, rms_eps=1e-6)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mk.lib()


def _run_layer(cfg, case, w, x):
    B = len(case.context_lens)
    kp, vp = bits_to_dev(case.k_pool), bits_to_dev(case.v_pool)
    wd = {n: bits_to_dev(a) for n, a in w.items()}
    xd = bits_to_dev(x)
    xo = torch.empty_like(xd)
    table = torch.from_numpy(case.block_table).to(DEV)
    ctx = torch.from_numpy(case.context_lens).to(DEV)
    mbps, max_ctx = case.block_table.shape[1], int(case.context_lens.max())
    pool = mk.mi_kv_pool_init(case.num_blocks, 16, cfg.num_kv_heads, cfg.head_dim, kp, vp)
    try:
        lc = mk.layer_config(cfg.hidden, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                             cfg.intermediate, cfg.rms_eps, cfg.rope_theta)
        lw = mk.layer_weights(**wd)
        need = mk.mi_decoder_layer_workspace_bytes(lc, pool, B, max_ctx)
        assert need > 0
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        mk.mi_decoder_layer_decode(pool, lc, lw, xd, xo, table, mbps, ctx, B, max_ctx, ws, need)
        torch.cuda.synchronize()
        assert mk.mi_kv_pool_check_errors(pool) == 0
    finally:
        mk.mi_kv_pool_destroy(pool)
    return dev_to_bits(xo), dev_to_bits(kp), dev_to_bits(vp)


def _oracle(cfg, case, w, x):
    return olayer.decoder_layer_decode(x, w, case.k_pool, case.v_pool, case.block_table,
                                       case.context_lens, cfg.block_size, cfg.num_q_heads,
                                       cfg.num_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.rope_theta,
                                       return_intermediates=True)


def _ordered(bits):
    """Monotone integer order of finite bf16 bit patterns."""
    x = np.asarray(bits, np.uint16).astype(np.int64)
    return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)


def _check_cache(case, cfg, gk, gv, inter, w):
    """Written slots vs the oracle. The device projects k and v with fp32
    accumulation and rounds once to bf16 (K after the float64 rotation), the
    oracle rounds the exact float64 value once. The check: every stored value
    is the bf16 rounding (nearest, ties to even) of some value within E of the
    exact one, with E = 2^-20 (sum_k |r1_k w_k| + |y|) per projected element (a
    bound of the fp32 accumulation and RMS-scale errors, ~16x the typical
    error) and, for K, the sum of the E of both rotation partners. So a value
    is bit-exact unless the exact value lies within E of a rounding boundary,
    and then at most one ulp off. Every other slot is untouched."""
    B = len(case.context_lens)
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    slots = np.zeros(case.k_pool.shape[:3], dtype=bool)
    for b, ctx in enumerate(case.context_lens):
        slots[case.block_table[b, ctx // 16], :, ctx % 16] = True
    sel = slots[..., None].repeat(D, -1)
    assert np.array_equal(gk[~sel], case.k_pool[~sel])
    assert np.array_equal(gv[~sel], case.v_pool[~sel])
    W = obf16.decode(w["w_qkv"])
    E = 2.0 ** -20 * (np.abs(inter["r1"]) @ np.abs(W).T + np.abs(inter["qkv"]))
    qkv = inter["qkv"]
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(B, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(B, Hkv, D)
    ek = E[:, Hq * D:(Hq + Hkv) * D].reshape(B, Hkv, D)
    ev = E[:, (Hq + Hkv) * D:].reshape(B, Hkv, D)
    ek = ek + np.roll(ek, D // 2, axis=-1)
    inexact = 0
    for b in range(B):
        pos = int(case.context_lens[b])
        blk, off = case.block_table[b, pos // 16], pos % 16
        for g in range(Hkv):
            for got, y, e, name in ((gk[blk, g, off], orope.apply(k[b, g], pos, cfg.rope_theta), ek[b, g], "K"),
                                    (gv[blk, g, off], v[b, g], ev[b, g], "V")):
                o = _ordered(got)
                lo, hi = _ordered(obf16.encode(y - e)), _ordered(obf16.encode(y + e))
                ok = (lo <= o) & (o <= hi)
                assert ok.all(), "%s b=%d g=%d dim %d: got %r, exact %r, E %r" % (
                    name, b, g, int(np.argmin(ok)), got[~ok][:3], y[~ok][:3], e[~ok][:3])
                inexact += int((got != obf16.encode(y)).sum())
    print("  cache: %d of %d written values not the exact value's rounding" % (inexact, 2 * B * Hkv * D),
          flush=True)


@pytest.mark.parametrize("cfg,std", [(SMALL, 0.05), (WIDE, 0.05), (MAXB, 0.02), (MAXB, 0.05),
                                     (MID, 0.03), (ONE, 0.05), (B17, 0.05)],
                         ids=["small", "wide_b20", "max_b32_g8", "max_b32_g8_std05", "mid_b12",
                              "one_b1", "b17"])
def test_layer_small_shapes(cfg, std):
    print("layer", cfg.name, flush=True)
    case = workloads.make_decode_case(cfg, pool="poison")
    w = workloads.make_layer_weights(cfg, std=std)
    x = workloads.make_layer_input(cfg)
    out, gk, gv = _run_layer(cfg, case, w, x)
    ref, _, _, inter = _oracle(cfg, case, w, x)
    mx, rel = check_tolerance(out, ref, cfg.name)
    print("  max|d| %.3g relL2 %.3g" % (mx, rel), flush=True)
    _check_cache(case, cfg, gk, gv, inter, w)


def test_layer_zero_output_projections_return_input_bit_exact():
    cfg = SMALL
    case = workloads.make_decode_case(cfg, pool="poison")
    w = dict(workloads.make_layer_weights(cfg, std=0.05))
    w["w_o"] = np.zeros_like(w["w_o"])
    w["w_down"] = np.zeros_like(w["w_down"])
    x = workloads.make_layer_input(cfg)
    out, _, _ = _run_layer(cfg, case, w, x)
    assert np.array_equal(out, x)


def test_layer_qwen3_8b_shape_full_size():
    """Qwen3-8B-shaped layer, batch 8, contexts U[512, 4096], full oracle."""
    cfg = workloads.CONFIGS["qwen3_8b_layer"]
    print("layer qwen3_8b_layer", flush=True)
    case = workloads.make_decode_case(cfg, pool="poison")
    w = workloads.make_layer_weights(cfg)
    x = workloads.make_layer_input(cfg)
    out, gk, gv = _run_layer(cfg, case, w, x)
    ref, _, _, inter = _oracle(cfg, case, w, x)
    mx, rel = check_tolerance(out, ref, "qwen3_8b_layer")
    print("  max|d| %.3g relL2 %.3g" % (mx, rel), flush=True)
    _check_cache(case, cfg, gk, gv, inter, w)


def test_layer_argument_errors():
    cfg = SMALL
    case = workloads.make_decode_case(cfg, pool="poison")
    kp, vp = bits_to_dev(case.k_pool), bits_to_dev(case.v_pool)
    pool = mk.mi_kv_pool_init(case.num_blocks, 16, cfg.num_kv_heads, cfg.head_dim, kp, vp)
    try:
        lc = mk.layer_config(300, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                             cfg.intermediate, cfg.rms_eps, cfg.rope_theta)
        assert mk.mi_decoder_layer_workspace_bytes(lc, pool, 3, 100) == 0     # hidden % 256
        lc = mk.layer_config(cfg.hidden, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                             cfg.intermediate, cfg.rms_eps, cfg.rope_theta)
        assert mk.mi_decoder_layer_workspace_bytes(lc, pool, 33, 100) == 0    # batch > 32
        need = mk.mi_decoder_layer_workspace_bytes(lc, pool, 3, 100)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        x = torch.zeros(3, cfg.hidden, dtype=torch.int16, device=DEV)
        lw = mk.layer_weights(*([x] * 7))
        with pytest.raises(mk.MikvError) as e:
            mk.mi_decoder_layer_decode(pool, lc, lw, x, x, x, 4, x, 3, 100, ws, need)
        assert e.value.status == mk.MI_ERR_INVALID_ARG                    # x_in aliases x_out
        with pytest.raises(mk.MikvError) as e:
            mk.mi_decoder_layer_decode(pool, lc, lw, x, x.clone(), x, 4, x, 3, 100, ws, need - 1)
        assert e.value.status == mk.MI_ERR_WORKSPACE_TOO_SMALL
    finally:
        mk.mi_kv_pool_destroy(pool)
