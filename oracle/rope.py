"""Rotary position embedding of cached keys, for pre-RoPE key quantization —
TEST INFRASTRUCTURE ONLY (see oracle/__init__).

The pages name the technique without defining it: KVQuant quantizes keys
before the rotary positional embedding is applied, so that the rotation does
not smear the channel structure the per-channel scales rely on ("Sub-8-Bit KV
Cache Quantization Is Not a Free Lever for an RDNA4 Agent Swarm", "What the
low-bit numbers actually cost"; the 3-bit row of its table; FAQ). The
embedding itself is the textbook one (RoFormer), with these readings, also
listed in the design notes:

  * frequencies theta_i = base^(-2 i / d) for i = 0 .. d/2 - 1 (base 10000
    unless configured);
  * channel pairs (i, i + d/2), the "rotate half" layout: at position t
        y_i       = x_i cos(t theta_i) - x_{i+d/2} sin(t theta_i)
        y_{i+d/2} = x_{i+d/2} cos(t theta_i) + x_i sin(t theta_i);
  * cached key t (0-based position in its sequence) is rotated by t inside
    attention, after dequantization; the query arrives already rotated by its
    own position.
Everything is float64. Parity of this part rests on the textbook definition,
not on the pages ("parity unpinned by the pages"); its pins are the
embedding's own properties (identity at position 0, a rotation of each pair,
dependence of q.k on the position difference only, composition, the complex
multiplication form).
"""
import numpy as np


def frequencies(d, base):
    """theta_i = base^(-2 i / d), i = 0 .. d/2 - 1, float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / d)


def rope(x, positions, base=10000.0):
    """Rotate vectors x [..., n, d] (float64) by their positions [n]."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(positions, np.float64)[:, None] * frequencies(d, base)[None, :]   # [n, d/2]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
