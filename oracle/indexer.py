"""Lightning indexer and top-k selector (oracle; test infrastructure).

[Notes §7] index score of query t against compressed block s:
    I_{t,s} = sum_h w^I_{t,h} * ReLU(q^I_{t,h} . K^IComp_s)
and the selected set  C^SprsComp_t = { C^Comp_s : I_{t,s} in Top-k(I_{t,:}) }.
[Notes §9] / [HF "Hybrid attention"]: the indexer's QK path runs in FP4, so
with MXFP4 keys the query heads are quantised to MXFP4 (groups of 32) before the
dot product; with f32 keys nothing is quantised.  Products of e2m1 values with
power-of-two scales are exact, so float64 gives the exact per-head dot.

Visibility (causality): query at absolute position p sees the compressed blocks
whose m tokens are all at or before p, i.e. blocks s < n_vis(p) =
min(floor((p+1)/m), cap); p < 0 sees none.

Top-k: the k' = min(k, n_vis) largest scores; ties go to the lower block
index; the result is listed in ascending block order and padded with -1 up to
k.  Scores are ranked in fp32 (the selector's score precision before the
BF16 variant of [Notes §9]).  The BF16 variant ([Notes §9]: the top-k
selector's index scores cut from FP32 to BF16): each fp32 score is rounded to
the nearest bf16 (ties to even) and the bf16 values are ranked, equal values
again going to the lower block index.
"""

import numpy as np

from .codecs import bf16_decode, bf16_encode, f32, idx_decode_rows, mxfp4_roundtrip


def n_visible(p, m, cap):
    if p < 0:
        return 0
    return int(min((p + 1) // m, cap))


def quantise_query(q, key_fmt):
    """q^I [..., H_I, d] -> the values the indexer multiplies (float64)."""
    q = f32(q).astype(np.float64)
    if key_fmt == "mxfp4":
        return mxfp4_roundtrip(q)
    return q


def index_scores(q_idx, w, keys, pos, m):
    """Scores for every (b, query) over its visible blocks.

    q_idx float [B][Q][H_I][d] (already decoded from bf16 where applicable),
    w [B][Q][H_I], keys: Idx, pos int [B][Q].
    Returns a list-of-lists of float64 arrays (length n_vis each).
    """
    B, Q, H, d = np.shape(q_idx)
    w = np.asarray(w, dtype=np.float64)
    out = []
    for b in range(B):
        row = []
        for t in range(Q):
            nv = n_visible(int(pos[b][t]), m, keys.cap)
            qh = quantise_query(np.asarray(q_idx)[b, t], keys.fmt)   # [H][d]
            K = idx_decode_rows(keys, b, np.arange(nv))               # [nv][d]
            dots = K @ qh.T                                           # [nv][H]
            row.append(np.maximum(dots, 0.0) @ w[b, t])
        out.append(row)
    return out


def ranked_scores(scores, score_dtype="f32"):
    """The values the selector ranks: the fp32 scores, or ("bf16") those
    rounded to the nearest bf16 (ties to even)."""
    s32 = f32(scores)
    if score_dtype == "bf16":
        return bf16_decode(bf16_encode(s32)) if len(s32) else s32.astype(np.float64)
    assert score_dtype == "f32"
    return s32.astype(np.float64)


def topk_from_scores(scores, k, score_dtype="f32"):
    """Ascending block ids of the k' largest ranked scores (lower id wins
    ties), padded with -1 to length k."""
    s = ranked_scores(scores, score_dtype)
    n = len(s)
    kk = min(k, n)
    order = sorted(range(n), key=lambda i: (-s[i], i))
    sel = sorted(order[:kk])
    return np.array(sel + [-1] * (k - kk), dtype=np.int64)


def index_topk(q_idx, w, keys, pos, m, k, score_dtype="f32"):
    scores = index_scores(q_idx, w, keys, pos, m)
    B = len(scores)
    Q = len(scores[0])
    out = np.full((B, Q, k), -1, dtype=np.int64)
    for b in range(B):
        for t in range(Q):
            out[b, t] = topk_from_scores(scores[b][t], k, score_dtype)
    return out, scores
