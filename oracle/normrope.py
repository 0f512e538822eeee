"""RMSNorm and partial RoPE around the core attention (oracle; test
infrastructure).

[Notes §9] (other CSA/HCA details):
  * Query / KV entry RMSNorm: before core attention, every query head and
    every compressed KV entry is RMS-normalised (this keeps the attention
    logits from blowing up);
  * Partial RoPE: RoPE is applied to the last 64 dims of the query, of the KV
    entry and of the core-attention output; since a compressed entry is both
    key and value, the output is rotated back by the query's position, which
    leaves it carrying relative position information.

Readings (the pages give no formulas; each is listed in the design notes):
  * RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma over all D dims of a head or
    entry, gamma a learned weight per dim, eps a parameter;
  * RoPE rotates adjacent pairs (x[2i], x[2i+1]) of the rotated dims by the
    angle pos * inv_freq[i] (the caller passes the inverse frequencies); the
    angle is the fp32 product fl32(fl32(pos) * inv_freq[i]) (what a kernel
    computes from an fp32 table), its sine and cosine exact;
  * the output correction rotates by -angle(query position);
  * a compressed entry's position is the last token of its block,
    i * m + m - 1 (the first position that sees it); a raw window token's is
    its own index.
"""

import numpy as np

from .codecs import f32


def rms_norm(x, gamma, eps):
    """x float [..., D] -> float64, normalised over the last axis."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(gamma, np.float64)


def rope_angles(pos, inv_freq):
    """pos int [...] -> float64 [..., n_pairs]: fl32(fl32(pos) * inv_freq)."""
    p = np.asarray(pos, np.float64).astype(np.float32)[..., None]
    inv = np.asarray(inv_freq, np.float32)
    return (p * inv).astype(np.float32).astype(np.float64)


def rope(x, pos, inv_freq, sign=1):
    """Rotate the last 2 * len(inv_freq) dims of x [..., D] in adjacent pairs by
    sign * angle(pos); pos broadcasts against x's leading axes."""
    x = np.array(x, np.float64, copy=True)
    n = len(inv_freq)
    a = rope_angles(pos, inv_freq) * sign                    # [..., n]
    c, s = np.cos(a), np.sin(a)
    r = x[..., x.shape[-1] - 2 * n:]
    x0, x1 = r[..., 0::2].copy(), r[..., 1::2].copy()
    r[..., 0::2] = x0 * c - x1 * s
    r[..., 1::2] = x0 * s + x1 * c
    x[..., x.shape[-1] - 2 * n:] = r
    return x


def entry_positions(blocks, m):
    """Position of compressed entry (block) i: its last token, i * m + m - 1."""
    return np.asarray(blocks, np.int64) * m + m - 1


def default_inv_freq(d_rope, base=10000.0):
    """The usual table fl32(base^(-2i/d_rope)); callers may pass any table."""
    i = np.arange(d_rope // 2, dtype=np.float64)
    return f32(base ** (-2.0 * i / d_rope))


def norm_rope(x, pos, nr):
    """The [Notes §9] steps of an `nr` option on rows x [..., D] at positions
    pos (broadcast against x's leading axes): RMSNorm when nr["gamma"] is not
    None, then RoPE when nr["inv_freq"] is not None (either step may be off,
    as in the library's calls)."""
    y = np.asarray(x, np.float64)
    if nr.get("gamma") is not None:
        y = rms_norm(y, nr["gamma"], nr["eps"])
    if nr.get("inv_freq") is not None:
        y = rope(y, pos, nr["inv_freq"])
    return y
