"""CSA / HCA core attention with the sliding-window branch (oracle; test infrastructure).

[Notes §7]: core attention is shared key-value MQA -- every query head attends
the same entries and each compressed entry is BOTH key and value (the full
D-dim entry, RoPE dims included).  The sliding-window branch lets each query
also see the most recent n_win uncompressed KV entries; [Notes §8] compress_ratio
table: they enter core attention together with the compressed entries, i.e.
one joint softmax (no de-duplication between the two sets).
[Notes §8]: HCA has no top-k -- every visible compressed entry is attended.
[Notes §9] attention sink: a learnable per-head logit z_h that joins the
softmax normaliser only, so total attention mass may be below 1.

For a query at absolute position p, head h:
  E  = selected compressed rows (CSA: top-k ids in [0, cap); HCA: s < n_vis(p))
       plus window tokens t in [max(0, p-n_win+1), p], read from ring row t mod R
  l_e = sm_scale * (q_h . v_e)
  M   = max(max_e l_e, z_h)          (z_h = -inf without a sink)
  out_h = sum_e exp(l_e - M) v_e / (sum_e exp(l_e - M) + exp(z_h - M))
  empty E and no sink -> out_h = 0.
Queries are decoded from bf16 (or taken as fp32); the output is rounded to bf16
(or fp32).  With `nr` (dict gamma, eps, inv_freq; [Notes §9] query RMSNorm and
partial RoPE, see normrope.py) each query head is RMS-normalised, its last
2 * len(inv_freq) dims rotated by the query position and the result rounded to
bf16 (the precision the attention multiplies in), and the output's same dims
are rotated back by the query position before the final rounding.
"""

import numpy as np

from .codecs import bf16_decode, bf16_encode, f32, kv_decode_rows
from .indexer import n_visible
from .normrope import norm_rope, rope


def window_positions(p, n_win):
    if p < 0 or n_win <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.arange(max(0, p - n_win + 1), p + 1, dtype=np.int64)


def _attend_one(qh, V, sm_scale, sink):
    """qh [H][D] float64, V [n][D] float64 -> [H][D] float64."""
    H, D = qh.shape
    if V.shape[0] == 0:
        return np.zeros((H, D))           # empty set: the weighted sum is 0
    logits = sm_scale * (qh @ V.T)        # [H][n]
    M = logits.max(axis=1)
    if sink is not None:
        M = np.maximum(M, sink)
    P = np.exp(logits - M[:, None])
    den = P.sum(axis=1)
    if sink is not None:
        den = den + np.exp(sink - M)
    return (P @ V) / den[:, None]


def _decode_q(q, q_fmt):
    if q_fmt == "bf16":
        return bf16_decode(q)
    return f32(q).astype(np.float64)


def _round_out(o, out_fmt):
    if out_fmt == "bf16":
        return bf16_encode(f32(o))
    return f32(o)


def _entries(comp, win, b, p, rows_comp, n_win):
    parts = []
    if len(rows_comp):
        parts.append(kv_decode_rows(comp, b, rows_comp))
    wp = window_positions(p, n_win)
    if len(wp):
        parts.append(kv_decode_rows(win, b, wp % win.cap))
    D = comp.d_nope + comp.d_rope
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, D))


def _prep_q(qd, pos, nr):
    """[Notes §9] query RMSNorm + partial RoPE, rounded to bf16 (see module doc)."""
    if nr is None:
        return qd
    pos = np.asarray(pos, np.int64)
    qn = norm_rope(qd, pos[:, :, None], nr)
    return bf16_decode(bf16_encode(f32(qn)))


def _post_out(out, pos, nr):
    if nr is None or nr.get("inv_freq") is None:
        return out
    return rope(out, np.asarray(pos, np.int64)[:, :, None], nr["inv_freq"], sign=-1)


def csa_attend(q, q_fmt, comp, topk, win, n_win, pos, sink, sm_scale, out_fmt, nr=None):
    """q [B][Q][H][D] (bf16 bits or f32), topk int [B][Q][k] (ids outside
    [0, cap) are skipped), pos int [B][Q], sink None | [H]."""
    qd = _prep_q(_decode_q(q, q_fmt), pos, nr)
    B, Q, H, D = qd.shape
    out = np.zeros((B, Q, H, D))
    sk = None if sink is None else np.asarray(sink, np.float64)
    for b in range(B):
        for t in range(Q):
            ids = np.asarray(topk[b][t], dtype=np.int64)
            ids = ids[(ids >= 0) & (ids < comp.cap)]
            V = _entries(comp, win, b, int(pos[b][t]), ids, n_win)
            out[b, t] = _attend_one(qd[b, t], V, sm_scale, sk)
    out = _post_out(out, pos, nr)
    return _round_out(out, out_fmt), out


def hca_attend(q, q_fmt, comp, m, win, n_win, pos, sink, sm_scale, out_fmt, nr=None):
    qd = _prep_q(_decode_q(q, q_fmt), pos, nr)
    B, Q, H, D = qd.shape
    out = np.zeros((B, Q, H, D))
    sk = None if sink is None else np.asarray(sink, np.float64)
    for b in range(B):
        for t in range(Q):
            p = int(pos[b][t])
            ids = np.arange(n_visible(p, m, comp.cap), dtype=np.int64)
            V = _entries(comp, win, b, p, ids, n_win)
            out[b, t] = _attend_one(qd[b, t], V, sm_scale, sk)
    out = _post_out(out, pos, nr)
    return _round_out(out, out_fmt), out
