"""Full decoder-layer decode step (test infrastructure only).

Course project, section 2.1, lists the pieces of a Qwen-style decoder layer:
RMSNorm (torch.nn.functional.rms_norm is allowed), RoPE, QKV projection with
grouped-query attention, a SwiGLU MLP (gate_proj / up_proj / down_proj with
SiLU), and the layer assembled with residual connections and two norms. The
pages do not write the assembly out; the reading taken is the pre-norm layer
of the Qwen models they run:

    r1  = RMSNorm(x) * w1
    qkv = r1 W_qkv^T               rows of W_qkv: q (Hq*D), k (Hkv*D), v (Hkv*D)
    write_decode_kv at pos = ctx   (cache stores bf16 RoPE(k) and bf16 v)
    o   = paged GQA decode attention of RoPE(q) over L = ctx + 1 tokens
    x2  = x + o W_o^T
    r2  = RMSNorm(x2) * w2
    a   = silu(r2 W_g^T) * (r2 W_u^T)
    out = x2 + a W_d^T

Weights use the nn.Linear layout [out_features, in_features] (y = x W^T).
Everything is float64; the only roundings are the cache stores (bf16, or the
E4M3 codes of those bf16 values for an 8-bit cache).
"""
import numpy as np

from . import attention
from . import bf16
from . import fp8
from . import paged
from . import rope


def rms_norm(x, w, eps):
    """y = x / sqrt(mean(x^2) + eps) * w over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(r, w_gate, w_up, w_down):
    """down(silu(gate(r)) * up(r)) with nn.Linear-layout weights (float64)."""
    return (silu(r @ w_gate.T) * (r @ w_up.T)) @ w_down.T


def decoder_layer_decode(x_bits, weights, k_pool, v_pool, block_table, context_lens,
                         block_size, num_q_heads, num_kv_heads, head_dim,
                         rms_eps, theta, return_intermediates=False, kv_scales=None):
    """One decode step of one layer for a batch of sequences.

    x_bits  : uint16 bf16 bits [B, H]
    weights : dict of uint16 bf16 bits: ln1_w [H], w_qkv [(Hq+2Hkv)D, H],
              w_o [H, Hq D], ln2_w [H], w_gate [I, H], w_up [I, H], w_down [H, I]
    k_pool, v_pool : uint16 [N, Hkv, bs, D] (not modified); with kv_scales =
              (k_scales [Hkv], v_scales [Hkv]) they are uint8 E4M3 codes of an
              8-bit cache: the stores become fp8.quantize of the bf16 values
              and the attention reads fp8.dequantize (vLLM-based
              inference-framework report, "FP8 KV Cache quantisation").
    Returns (out_f64 [B, H], k_pool_new, v_pool_new[, intermediates]).
    """
    x = bf16.decode(x_bits)
    W = {name: bf16.decode(val) for name, val in weights.items()}
    B, H = x.shape
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    G = Hq // Hkv

    r1 = rms_norm(x, W["ln1_w"], rms_eps)
    qkv = r1 @ W["w_qkv"].T
    q = qkv[:, : Hq * D].reshape(B, Hq, D)
    k = qkv[:, Hq * D: (Hq + Hkv) * D].reshape(B, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(B, Hkv, D)

    f8 = kv_scales is not None
    k_new = np.array(k_pool, dtype=np.uint8 if f8 else np.uint16, copy=True)
    v_new = np.array(v_pool, dtype=np.uint8 if f8 else np.uint16, copy=True)
    q_rot = np.empty_like(q)
    for b in range(B):
        pos = int(context_lens[b])
        blk, off = paged.slot(block_table[b], pos, block_size)
        for g in range(Hkv):
            kb = bf16.encode(rope.apply(k[b, g], pos, theta))
            vb = bf16.encode(v[b, g])
            if f8:
                k_new[blk, g, off] = fp8.quantize(bf16.decode(kb), kv_scales[0][g])
                v_new[blk, g, off] = fp8.quantize(bf16.decode(vb), kv_scales[1][g])
            else:
                k_new[blk, g, off] = kb
                v_new[blk, g, off] = vb
        q_rot[b] = rope.apply(q[b], pos, theta)

    o = np.empty((B, Hq, D), dtype=np.float64)
    scale = 1.0 / np.sqrt(np.float64(D))
    for b in range(B):
        L = int(context_lens[b]) + 1
        for g in range(Hkv):
            ks, vs = attention.gather_kv(k_new, v_new, block_table, block_size, b, g, L)
            if f8:
                K = fp8.dequantize(ks, kv_scales[0][g])
                V = fp8.dequantize(vs, kv_scales[1][g])
            else:
                K, V = bf16.decode(ks), bf16.decode(vs)
            for h in range(g * G, (g + 1) * G):
                o[b, h] = attention.attend(q_rot[b, h], K, V, scale)

    x2 = x + o.reshape(B, Hq * D) @ W["w_o"].T
    r2 = rms_norm(x2, W["ln2_w"], rms_eps)
    out = x2 + swiglu(r2, W["w_gate"], W["w_up"], W["w_down"])
    if return_intermediates:
        inter = dict(r1=r1, qkv=qkv, q_rot=q_rot, o=o, x2=x2, r2=r2)
        return out, k_new, v_new, inter
    return out, k_new, v_new
