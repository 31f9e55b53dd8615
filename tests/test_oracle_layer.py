"""Pins for the oracle's decoder layer (CPU only): library routines the course
project names (rms_norm, silu, scaled_dot_product_attention), closed forms
and special cases that switch parts of the layer off."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads
from oracle import attention, bf16, layer, rope

SMALL = workloads.DecodeConfig(
    "small_layer", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=16,
    num_blocks=64, rope_theta=1e4, ctx_draw="fixed", ctx_fixed=(0, 20, 47), seed=11,
    hidden=64, intermediate=96, rms_eps=1e-6)


def _inputs(cfg=SMALL, std=0.2):
    case = workloads.make_decode_case(cfg, pool="poison")
    w = workloads.make_layer_weights(cfg, std=std)
    x = workloads.make_layer_input(cfg)
    return case, w, x


def _run(case, w, x, cfg=SMALL, **kw):
    return layer.decoder_layer_decode(x, w, case.k_pool, case.v_pool, case.block_table,
                                      case.context_lens, cfg.block_size, cfg.num_q_heads,
                                      cfg.num_kv_heads, cfg.head_dim, cfg.rms_eps,
                                      cfg.rope_theta, **kw)


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    x, w = rng.standard_normal((7, 4096)), rng.standard_normal(4096)
    ref = F.rms_norm(torch.from_numpy(x), (4096,), torch.from_numpy(w), eps=1e-6).numpy()
    assert np.allclose(layer.rms_norm(x, w, 1e-6), ref, rtol=1e-14, atol=1e-14)


def test_rms_norm_constant_input_closed_form():
    for c in [0.0, 1e-4, 1.0, 37.5]:
        y = layer.rms_norm(np.full((2, 128), c), np.full(128, 2.0), 1e-6)
        assert np.allclose(y, 2.0 * c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)


def test_silu_matches_torch_and_limits():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(layer.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)
    assert layer.silu(np.array([0.0]))[0] == 0.0
    assert abs(layer.silu(np.array([50.0]))[0] - 50.0) < 1e-12


def test_layer_matches_torch_library_composition():
    """The whole layer rebuilt from torch fp64 library routines: rms_norm,
    linear, sdpa(enable_gqa), silu."""
    cfg = SMALL
    case, w, x = _inputs()
    out, kn, vn, inter = _run(case, w, x, return_intermediates=True)
    W = {k: torch.from_numpy(bf16.decode(v)) for k, v in w.items()}
    xt = torch.from_numpy(bf16.decode(x))
    B, Hq, Hkv, D = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    r1 = F.rms_norm(xt, (cfg.hidden,), W["ln1_w"], eps=cfg.rms_eps)
    qkv = F.linear(r1, W["w_qkv"])
    assert np.allclose(qkv.numpy(), inter["qkv"], rtol=0, atol=1e-12)
    o = torch.empty(B, Hq * D, dtype=torch.float64)
    for b in range(B):
        L = int(case.context_lens[b]) + 1
        idx = [(int(case.block_table[b, p // 16]), p % 16) for p in range(L)]
        K = torch.from_numpy(bf16.decode(np.stack([kn[blk, :, off] for blk, off in idx], 1)))
        V = torch.from_numpy(bf16.decode(np.stack([vn[blk, :, off] for blk, off in idx], 1)))
        qr = torch.from_numpy(inter["q_rot"][b])[None, :, None, :]
        o[b] = F.scaled_dot_product_attention(qr, K[None], V[None], enable_gqa=True)[0, :, 0, :].reshape(-1)
    x2 = xt + F.linear(o, W["w_o"])
    r2 = F.rms_norm(x2, (cfg.hidden,), W["ln2_w"], eps=cfg.rms_eps)
    ref = x2 + F.linear(F.silu(F.linear(r2, W["w_gate"])) * F.linear(r2, W["w_up"]), W["w_down"])
    assert np.allclose(out, ref.numpy(), rtol=0, atol=1e-11)


def test_layer_cache_write_is_rounded_rope_of_projection():
    cfg = SMALL
    case, w, x = _inputs()
    out, kn, vn, inter = _run(case, w, x, return_intermediates=True)
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    for b, ctx in enumerate(case.context_lens):
        blk, off = case.block_table[b, ctx // 16], ctx % 16
        k = inter["qkv"][b, Hq * D:(Hq + Hkv) * D].reshape(Hkv, D)
        v = inter["qkv"][b, (Hq + Hkv) * D:].reshape(Hkv, D)
        assert np.array_equal(kn[blk, :, off], bf16.encode(rope.apply(k, int(ctx), cfg.rope_theta)))
        assert np.array_equal(vn[blk, :, off], bf16.encode(v))


def test_layer_zero_output_projections_return_input_exactly():
    case, w, x = _inputs()
    w = dict(w)
    w["w_o"] = np.zeros_like(w["w_o"])
    w["w_down"] = np.zeros_like(w["w_down"])
    out, _, _ = _run(case, w, x)
    assert np.array_equal(out, bf16.decode(x))


def test_layer_zero_gate_leaves_attention_residual():
    cfg = SMALL
    case, w, x = _inputs()
    w = dict(w)
    w["w_gate"] = np.zeros_like(w["w_gate"])           # silu(0) = 0 kills the MLP
    out, _, _, inter = _run(case, w, x, return_intermediates=True)
    assert np.array_equal(out, inter["x2"])
    o = inter["o"].reshape(cfg.batch, -1)
    assert np.allclose(inter["x2"], bf16.decode(x) + o @ bf16.decode(w["w_o"]).T, rtol=0, atol=1e-13)


def test_layer_sampled_rows_fsum_brute_force():
    """QKV, o_proj and SwiGLU products checked elementwise with math.fsum."""
    cfg = SMALL
    case, w, x = _inputs()
    out, _, _, inter = _run(case, w, x, return_intermediates=True)
    Wq = bf16.decode(w["w_qkv"])
    Wd, Wg, Wu = bf16.decode(w["w_down"]), bf16.decode(w["w_gate"]), bf16.decode(w["w_up"])
    b = 1
    for n in [0, 5, 63, 64, 100, 127]:
        ref = math.fsum(inter["r1"][b, i] * Wq[n, i] for i in range(cfg.hidden))
        assert abs(inter["qkv"][b, n] - ref) < 1e-13
    r2 = inter["r2"][b]
    a = [0.0] * cfg.intermediate
    for j in range(cfg.intermediate):
        g = math.fsum(r2[i] * Wg[j, i] for i in range(cfg.hidden))
        u = math.fsum(r2[i] * Wu[j, i] for i in range(cfg.hidden))
        a[j] = g / (1.0 + math.exp(-g)) * u
    for n in [0, 17, 63]:
        ref = inter["x2"][b, n] + math.fsum(a[j] * Wd[n, j] for j in range(cfg.intermediate))
        assert abs(out[b, n] - ref) < 1e-12


def test_layer_position_zero_sequence_attends_to_itself_only():
    """ctx = 0: attention returns the sequence's own (bf16-rounded) v."""
    cfg = SMALL
    case, w, x = _inputs()
    out, kn, vn, inter = _run(case, w, x, return_intermediates=True)
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    v = bf16.decode(bf16.encode(inter["qkv"][0, (Hq + Hkv) * D:].reshape(Hkv, D)))
    G = Hq // Hkv
    for h in range(Hq):
        assert np.array_equal(inter["o"][0, h], v[h // G])


def test_layer_with_8bit_cache_composes_the_pinned_fp8_write_and_attention():
    """An 8-bit cache changes only the stores and the reads: the projections
    equal the bf16 layer's; the new slots hold fp8.quantize of the bf16 layer's
    stored K and V; the attention output equals paged_gqa_decode_fp8 (pinned
    against the bf16 attention) over the new codes."""
    from oracle import fp8
    cfg = SMALL
    case = workloads.make_decode_case(cfg, pool="poison", kv_format="fp8")
    w = workloads.make_layer_weights(cfg, std=0.2)
    x = workloads.make_layer_input(cfg)
    ks = np.array([0.75, 1.5], np.float32)
    vs = np.array([2.0, 0.3], np.float32)
    out8, k8, v8, i8 = _run(case, w, x, return_intermediates=True, kv_scales=(ks, vs))
    zeros = np.zeros(case.k_pool.shape, np.uint16)
    case16 = workloads.make_decode_case(cfg, pool="poison")
    _, kb, vb, ib = layer.decoder_layer_decode(
        x, w, zeros, zeros.copy(), case16.block_table, case16.context_lens, 16, cfg.num_q_heads,
        cfg.num_kv_heads, cfg.head_dim, cfg.rms_eps, cfg.rope_theta, return_intermediates=True)
    assert np.array_equal(case.block_table, case16.block_table)
    for name in ("r1", "qkv", "q_rot"):
        assert np.array_equal(i8[name], ib[name])
    written = np.zeros(case.k_pool.shape[:3], bool)
    for b, ctx in enumerate(case.context_lens):
        blk, off = case.block_table[b, ctx // 16], ctx % 16
        written[blk, :, off] = True
        for g in range(cfg.num_kv_heads):
            assert np.array_equal(k8[blk, g, off], fp8.quantize(bf16.decode(kb[blk, g, off]), ks[g]))
            assert np.array_equal(v8[blk, g, off], fp8.quantize(bf16.decode(vb[blk, g, off]), vs[g]))
    assert np.array_equal(k8[~written], case.k_pool[~written])
    o = attention.paged_gqa_decode_fp8(i8["q_rot"], k8, v8, case.block_table, case.context_lens,
                                       16, ks, vs, q_is_bits=False)
    assert np.array_equal(i8["o"], o)
