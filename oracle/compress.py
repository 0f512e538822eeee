"""Token-level KV compressor (oracle; test infrastructure).

[Notes §8] (HCA) gives the non-overlap compressor exactly:
    S_{m'i : m'(i+1)-1} = Softmax_row(Z_{m'i : m'(i+1)-1} + B)
    C^Comp_i = sum_{j=m'i}^{m'(i+1)-1} S_j (elementwise) C_j
with learned positional bias B (one row per in-block slot).  The product is
elementwise, so gate, bias and softmax weights are per channel and the softmax
runs over the rows (slots) of the block, independently for every channel.

[Notes §7] (CSA) has two KV streams C_a, C_b and two gate streams Z_a, Z_b, and
each compressed entry pools 2m adjacent entries with row-wise softmax weights,
adjacent entries overlapping; [HF "Hybrid attention"] calls it softmax-gated
pooling with a learned positional bias.  Reading adopted (the pages give no
formula): entry i pools the m "previous-role" rows of block i-1 (stream a)
and the m "current-role" rows of block i (stream b) under ONE softmax over the
2m slots, with bias rows ordered [prev slot 0..m-1, cur slot 0..m-1]; block 0
has no previous block, its prev slots are excluded (weight 0).  This pairing
is "parity unpinned" by the pages.

Inputs of one call cover tokens [t0, t0+T) (t0 and T multiples of m):
  kv_cur, gate_cur   [B][T][d]  rows = tokens t0 .. t0+T-1 (stream b / only stream)
  kv_prev, gate_prev [B][T][d]  rows = tokens t0-m .. t0+T-m-1 (stream a), or None
  pos_bias           [slots][d] (slots = 2m with overlap, m without), or None = 0
  gate None means all-zero gate logits.
With `nr` (dict gamma, eps, inv_freq; [Notes §9] KV entry RMSNorm and
partial RoPE, see normrope.py) each pooled fp32 row is RMS-normalised and its
last 2 * len(inv_freq) dims rotated by the entry's position (its block's last
token), then rounded to fp32 again.
Output: float64 [B][T/m][d], rounded to fp32 -- compressed entries t0/m ...
"""

import numpy as np

from .codecs import f32
from .normrope import entry_positions, norm_rope


def _softmax_rows(logits):
    """Softmax over axis -2 (the slots), with max subtraction; -inf = excluded."""
    mx = np.max(logits, axis=-2, keepdims=True)
    e = np.exp(logits - mx)
    return e / np.sum(e, axis=-2, keepdims=True)


def compress(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, m, t0, nr=None):
    y = _pool(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, m, t0)
    if nr is None:
        return y
    nb = y.shape[1]
    blocks = t0 // m + np.arange(nb)
    y = norm_rope(y, entry_positions(blocks, m)[None, :], nr)
    return f32(y).astype(np.float64)


def _pool(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, m, t0):
    kv_cur = np.asarray(kv_cur, dtype=np.float64)
    B, T, d = kv_cur.shape
    assert T % m == 0 and t0 % m == 0
    nb = T // m
    g_cur = np.zeros_like(kv_cur) if gate_cur is None else np.asarray(gate_cur, np.float64)
    overlap = kv_prev is not None
    slots = 2 * m if overlap else m
    bias = np.zeros((slots, d)) if pos_bias is None else np.asarray(pos_bias, np.float64)
    assert bias.shape == (slots, d)

    cur_c = kv_cur.reshape(B, nb, m, d)
    cur_z = g_cur.reshape(B, nb, m, d) + bias[None, None, slots - m:, :]
    if not overlap:
        S = _softmax_rows(cur_z)
        y = np.sum(S * cur_c, axis=-2)
        return f32(y).astype(np.float64)

    kv_prev = np.asarray(kv_prev, dtype=np.float64)
    g_prev = np.zeros_like(kv_prev) if gate_prev is None else np.asarray(gate_prev, np.float64)
    prev_c = kv_prev.reshape(B, nb, m, d)
    prev_z = g_prev.reshape(B, nb, m, d) + bias[None, None, :m, :]
    if t0 == 0:
        # global block 0 has no previous block: its prev slots are excluded
        prev_z = prev_z.copy()
        prev_z[:, 0] = -np.inf
        prev_c = prev_c.copy()
        prev_c[:, 0] = 0.0
    C = np.concatenate([prev_c, cur_c], axis=-2)      # [B][nb][2m][d]
    Z = np.concatenate([prev_z, cur_z], axis=-2)
    S = _softmax_rows(Z)
    y = np.sum(S * C, axis=-2)
    return f32(y).astype(np.float64)
