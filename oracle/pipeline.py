"""One CSA layer and one HCA layer chained from the four operations (oracle;
test infrastructure).

[Notes §8] compress_ratio table: ratio 4 = CSA (overlap compressor, lightning
indexer top-k, then core attention over the selected compressed entries
together with the sliding-window uncompressed entries); ratio 128 = HCA
(non-overlap compressor, no top-k, dense over all compressed entries plus the
window); ratio 0 = window only.
"""

import numpy as np

from .attend import csa_attend, hca_attend
from .codecs import KV, f32, idx_encode, kv_encode
from .compress import compress
from .indexer import index_topk


def csa_layer(q, q_fmt, q_idx, w, comp, keys, win, n_win, pos, m, k, sm_scale,
              sink=None, out_fmt="bf16"):
    topk, scores = index_topk(q_idx, w, keys, pos, m, k)
    out_bits, out = csa_attend(q, q_fmt, comp, topk, win, n_win, pos, sink, sm_scale, out_fmt)
    return dict(topk=topk, scores=scores, out=out_bits, out_f64=out)


def hca_layer(q, q_fmt, comp, m, win, n_win, pos, sm_scale, sink=None, out_fmt="bf16"):
    out_bits, out = hca_attend(q, q_fmt, comp, m, win, n_win, pos, sink, sm_scale, out_fmt)
    return dict(out=out_bits, out_f64=out)


def workload1(g, k=64, n_win=128, m=4, d_nope=64):
    """fp32 full CSA pipeline from raw token streams (workload 1).

    The attention entries pool (kv_a, z_a) as the previous role and (kv_b, z_b)
    as the current role; the index keys pool (ki_a, zi_a) / (ki_b, zi_b) the
    same way; the window ring holds the last n_win raw kv_b rows.
    """
    B, T, D = g["kv_b"].shape
    # prev-role rows of a call starting at t0 = 0 are tokens -m .. T-m-1
    prev = lambda x: np.concatenate([np.zeros_like(x[:, :m]), x[:, :T - m]], axis=1)
    y = compress(g["kv_b"], g["z_b"], prev(g["kv_a"]), prev(g["z_a"]), g["bias"], m, 0)
    yi = compress(g["ki_b"], g["zi_b"], prev(g["ki_a"]), prev(g["zi_a"]), g["bias_i"], m, 0)
    comp = kv_encode(y, "f32", d_nope)
    keys = idx_encode(yi, "f32")
    R = n_win
    rows = np.arange(T - R, T) % R
    ring = np.empty((B, R, D), dtype=np.float32)
    ring[:, rows] = f32(g["kv_b"][:, T - R:])
    win = kv_encode(ring, "f32", d_nope)
    res = csa_layer(g["q"], "f32", g["q_idx"], g["w"], comp, keys, win, n_win,
                    g["pos"], m, k, D ** -0.5, None, "f32")
    res.update(comp=comp, keys=keys, win=win, y=y, yi=yi)
    return res


def _ring(pre, tokens, t_first, R):
    """Raw-token ring of R rows: pre holds tokens t_first - len(pre) .. t_first - 1,
    tokens holds t_first .. t_first + T - 1; token t sits at row t mod R (rows
    never written stay zero)."""
    B, _, D = tokens.shape
    ring = np.zeros((B, R, D), dtype=np.float32)
    npre = pre.shape[1]
    for i in range(npre):
        ring[:, (t_first - npre + i) % R] = pre[:, i]
    for j in range(tokens.shape[1]):
        ring[:, (t_first + j) % R] = tokens[:, j]
    return ring


def prefill_caches(g, m_csa=4, m_hca=128, n_win=128, d_nope=448):
    """Caches of one CSA and one HCA layer after a prefill chunk (workload 5).

    The cached context is cache-direct (entries and keys as given); the chunk
    [ctx, ctx + T) is pooled by the compressors ([Notes §7] overlap for CSA
    entries and indexer keys, [Notes §8] non-overlap for HCA) and appended.
    The raw-token window rings hold tokens ctx - n_win + 1 .. ctx + T - 1 in
    R = T + n_win rows (row = token mod R), so every query of the chunk finds
    its whole window.
    """
    ctx = int(g["pos"][0, 0])
    T = g["q"].shape[1]
    y = compress(g["csa_kv_cur"], g["csa_z_cur"], g["csa_kv_prev"], g["csa_z_prev"],
                 g["csa_bias"], m_csa, ctx)
    yi = compress(g["idx_kv_cur"], g["idx_z_cur"], g["idx_kv_prev"], g["idx_z_prev"],
                  g["idx_bias"], m_csa, ctx)
    yh = compress(g["hca_kv"], g["hca_z"], None, None, g["hca_bias"], m_hca, ctx)
    R = T + n_win
    out = dict(
        y=y, yi=yi, yh=yh, R=R,
        comp=kv_encode(np.concatenate([g["csa_comp"], f32(y)], axis=1), "fp8", d_nope),
        keys=idx_encode(np.concatenate([g["keys"], f32(yi)], axis=1), "mxfp4"),
        hcomp=kv_encode(np.concatenate([g["hca_comp"], f32(yh)], axis=1), "fp8", d_nope),
        win=kv_encode(_ring(g["csa_win_pre"], g["csa_kv_cur"], ctx, R), "fp8", d_nope),
        hwin=kv_encode(_ring(g["hca_win_pre"], g["hca_kv"], ctx, R), "fp8", d_nope),
    )
    return out
