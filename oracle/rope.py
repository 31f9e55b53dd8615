"""Rotary position embedding (test infrastructure only).

Course project, section 2.1, lists "construction and application of RoPE" as
a component; the pages give no formula. Readings (stated in full where the
oracle is documented):

* half-split pairing: dimension i pairs with i + D/2 (the convention of the
  Qwen models the pages run and compare token-for-token against);
* inverse frequencies inv_freq_i = theta^(-2i/D), i < D/2, integer positions,
  no scaling;
* the new token's position is its logical index, i.e. the number of tokens
  cached before it.

All arithmetic is float64.
"""
import numpy as np


def inv_freq(head_dim, theta):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / head_dim)


def angles(pos, head_dim, theta):
    """a_i = pos * inv_freq_i, float64."""
    return np.float64(pos) * inv_freq(head_dim, theta)


def apply(x, pos, theta):
    """Rotate the last axis of ``x`` (float64, length D) to position ``pos``.

    y_i       = x_i cos a_i - x_{i+D/2} sin a_i
    y_{i+D/2} = x_{i+D/2} cos a_i + x_i sin a_i
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("head_dim must be even")
    h = d // 2
    a = angles(pos, d, theta)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :h], x[..., h:]
    y = np.empty_like(x)
    y[..., :h] = x1 * c - x2 * s
    y[..., h:] = x2 * c + x1 * s
    return y
