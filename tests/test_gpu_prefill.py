"""GPU parity for chunked prefill (many queries per sequence): the
query-tiled FP4 index scan, then CSA / HCA attention of every chunk query,
against the CPU oracle on identical input bytes.  Small cases cover every
query; the full 1M-context chunk of 4096 queries is checked on sampled
queries (the oracle computes those one by one)."""

import numpy as np
import pytest
import torch

from long_context_attention_v4attn_amd import synth
from oracle import codecs as C
from oracle.attend import csa_attend, hca_attend
from oracle.indexer import index_scores, index_topk
from oracle.pipeline import prefill_caches
from tests import parity as P
from tests.test_gpu_ops import _index_case, _rng

pytestmark = pytest.mark.gpu

STREAMS = ("csa_kv_cur", "csa_z_cur", "csa_kv_prev", "csa_z_prev", "idx_kv_cur", "idx_z_cur",
           "idx_kv_prev", "idx_z_prev", "hca_kv", "hca_z")


@pytest.mark.parametrize("Bn,Q,cap,k", [(1, 40, 5000, 300), (2, 11, 20000, 512), (1, 8, 16400, 64)])
def test_index_topk_query_tiled(lib, Bn, Q, cap, k):
    """Q >= 8 queries of a sequence with 16 index heads take the query-tiled
    scan: ragged query tiles, several block ranges, per-query visibility."""
    print(f"index query-tiled B={Bn} Q={Q} cap={cap} k={k}", flush=True)
    rng = _rng(Q * 31 + cap)
    m = 4
    pos = np.empty((Bn, Q), np.int64)
    for b in range(Bn):
        base = 4 * (cap - Q // 4 - 3) + b * 5
        pos[b] = base + np.arange(Q)
    pos[0, 0] = 4 * (k // 2)          # a query that sees fewer than k blocks
    pos[-1, -1] = 4 * cap + 40        # a query that sees the whole cache
    kinds = _index_case(lib, rng, Bn, Q, cap, 16, k, m, pos)
    assert kinds.count("exact") >= len(kinds) // 2


def _round_streams(g):
    """The chunk's token streams as bf16 (what the device receives), and the
    same values as fp32 for the oracle."""
    bits = {}
    for name in STREAMS:
        bits[name] = C.bf16_encode(g[name])
        g[name] = C.bf16_decode(bits[name]).astype(np.float32)
    return bits


def _bf16_t(bits):
    return P.dev(bits.view(np.int16)).view(torch.bfloat16)


def _prefill_case(ctx, chunk):
    c = synth.WORKLOADS[5]
    g = synth.prefill_inputs(5, ctx=ctx, chunk=chunk)
    bits = _round_streams(g)
    ref = prefill_caches(g, c["m_csa"], c["m_hca"], c["n_win"], c["d_nope"])
    return c, g, bits, ref


def test_prefill_chunk_compress(lib):
    """The chunk's CSA entries, indexer keys and HCA entries (GPU compress,
    t0 = ctx) against the oracle's, appended after the cached part."""
    c, g, bits, ref = _prefill_case(8192, 256)
    ctx, T = 8192, 256
    n_csa, n_hca = ctx // 4, ctx // 128
    D, dI = c["d_nope"] + c["d_rope"], c["d_I"]
    comp = lib.KVCache.empty(1, n_csa + T // 4, c["d_nope"], c["d_rope"], lib.KV_FP8_BF16ROPE)
    keys = lib.IdxCache.empty(1, n_csa + T // 4, dI, lib.IDX_MXFP4)
    hcomp = lib.KVCache.empty(1, n_hca + T // 128, c["d_nope"], c["d_rope"], lib.KV_FP8_BF16ROPE)
    lib.v4attn_compress(_bf16_t(bits["csa_kv_cur"]), _bf16_t(bits["csa_z_cur"]),
                        _bf16_t(bits["csa_kv_prev"]), _bf16_t(bits["csa_z_prev"]),
                        P.dev(g["csa_bias"]), 4, ctx, comp)
    lib.v4attn_compress(_bf16_t(bits["idx_kv_cur"]), _bf16_t(bits["idx_z_cur"]),
                        _bf16_t(bits["idx_kv_prev"]), _bf16_t(bits["idx_z_prev"]),
                        P.dev(g["idx_bias"]), 4, ctx, keys)
    lib.v4attn_compress(_bf16_t(bits["hca_kv"]), _bf16_t(bits["hca_z"]), None, None,
                        P.dev(g["hca_bias"]), 128, ctx, hcomp)
    torch.cuda.synchronize()
    back = P.kv_from_dev(comp)
    P.check_fp8_rows(_rows_kv(back, n_csa, n_csa + T // 4), ref["y"], c["d_nope"])
    bi = P.idx_from_dev(keys)
    P.check_mxfp4_rows(C.Idx("mxfp4", dI, bi.codes[:, n_csa:], bi.scales[:, n_csa:]), ref["yi"])
    hb = P.kv_from_dev(hcomp)
    P.check_fp8_rows(_rows_kv(hb, n_hca, n_hca + T // 128), ref["yh"], c["d_nope"])


def _rows_kv(kv, r0, r1):
    return C.KV(kv.fmt, kv.d_nope, kv.d_rope, kv.nope[:, r0:r1], kv.rope[:, r0:r1],
                kv.scale[:, r0:r1])


def _attend_inputs(lib, c, g, ref):
    D = c["d_nope"] + c["d_rope"]
    qb = C.bf16_encode(g["q"])
    return dict(q=_bf16_t(qb), qb=qb, comp=P.kv_to_dev(ref["comp"]), keys=P.idx_to_dev(ref["keys"]),
                hcomp=P.kv_to_dev(ref["hcomp"]), win=P.kv_to_dev(ref["win"]),
                hwin=P.kv_to_dev(ref["hwin"]), pos=P.dev(g["pos"]), sc=D ** -0.5)


def test_prefill_pair_small_every_query(lib):
    """A 256-token chunk after 8192 cached tokens: index top-k, CSA attend
    (oracle top-k as input) and HCA attend for every chunk query."""
    c, g, bits, ref = _prefill_case(8192, 256)
    k, n_win = 512, c["n_win"]
    x = _attend_inputs(lib, c, g, ref)
    qi = C.bf16_encode(g["q_idx"])
    qid = C.bf16_decode(qi).astype(np.float32)
    topk = lib.v4attn_index_topk(_bf16_t(qi), P.dev(g["w"]), x["keys"], x["pos"], 4, k)
    torch.cuda.synchronize()
    sc = index_scores(qid, g["w"], ref["keys"], g["pos"], 4)
    gt = topk.cpu().numpy()
    kinds = [P.check_topk_row(gt[0, t], sc[0][t], k) for t in range(gt.shape[1])]
    assert kinds.count("exact") >= len(kinds) // 2
    ref_topk, _ = index_topk(qid, g["w"], ref["keys"], g["pos"], 4, k)
    out = lib.v4attn_csa_attend(x["q"], x["comp"], P.dev(ref_topk.astype(np.int32)), x["win"],
                                n_win, x["pos"], None, x["sc"])
    hout = lib.v4attn_hca_attend(x["q"], x["hcomp"], 128, x["hwin"], n_win, x["pos"], None,
                                 x["sc"])
    torch.cuda.synchronize()
    _, r = csa_attend(x["qb"], "bf16", ref["comp"], ref_topk, ref["win"], n_win, g["pos"], None,
                      x["sc"], "bf16")
    P.check_out(P.out_to_f64(out), r, what="csa prefill")
    _, rh = hca_attend(x["qb"], "bf16", ref["hcomp"], 128, ref["hwin"], n_win, g["pos"], None,
                       x["sc"], "bf16")
    P.check_out(P.out_to_f64(hout), rh, what="hca prefill")


def test_prefill_pair_full_size_sampled(lib):
    """The 1M-context chunk of 4096 queries: every query computed on the GPU,
    sampled queries (both ends of query tiles and block ranges) checked."""
    c, g, bits, ref = _prefill_case(c_ctx := synth.WORKLOADS[5]["ctx"], synth.WORKLOADS[5]["chunk"])
    k, n_win = c["k"], c["n_win"]
    T = g["q"].shape[1]
    rows = np.array([0, 1, 7, 8, 2047, 2048, T - 1])
    print(f"prefill full size: ctx={c_ctx} chunk={T} sampled rows {rows.tolist()}", flush=True)
    x = _attend_inputs(lib, c, g, ref)
    qi = C.bf16_encode(g["q_idx"])
    qid = C.bf16_decode(qi).astype(np.float32)
    topk = lib.v4attn_index_topk(_bf16_t(qi), P.dev(g["w"]), x["keys"], x["pos"], 4, k)
    torch.cuda.synchronize()
    gt = topk.cpu().numpy()
    sc = index_scores(qid[:, rows], g["w"][:, rows], ref["keys"], g["pos"][:, rows], 4)
    for i, t in enumerate(rows):
        P.check_topk_row(gt[0, t], sc[0][i], k)
    ref_topk, _ = index_topk(qid[:, rows], g["w"][:, rows], ref["keys"], g["pos"][:, rows], 4, k)
    tk = gt.copy()
    tk[0, rows] = ref_topk[0]
    out = lib.v4attn_csa_attend(x["q"], x["comp"], P.dev(tk.astype(np.int32)), x["win"], n_win,
                                x["pos"], None, x["sc"])
    hout = lib.v4attn_hca_attend(x["q"], x["hcomp"], 128, x["hwin"], n_win, x["pos"], None,
                                 x["sc"])
    torch.cuda.synchronize()
    qs = x["qb"][:, rows]
    ps = g["pos"][:, rows]
    _, r = csa_attend(qs, "bf16", ref["comp"], ref_topk, ref["win"], n_win, ps, None, x["sc"], "bf16")
    P.check_out(P.out_to_f64(out)[:, rows], r, what="csa prefill 1M")
    _, rh = hca_attend(qs, "bf16", ref["hcomp"], 128, ref["hwin"], n_win, ps, None, x["sc"], "bf16")
    P.check_out(P.out_to_f64(hout)[:, rows], rh, what="hca prefill 1M")


# ---------------------------------------------------------------- sampled-threshold selection

def _planted_keys(n, sampled_score_shift, other_shift, seed):
    """MXFP4 keys that are all one random key r with every e8m0 scale byte
    raised by a shift: blocks of the sample tiles (block % 256 < 16) by
    `sampled_score_shift`, the others by `other_shift`.  A shift j multiplies
    the score by exactly 2^j (exact FP4 products, positively homogeneous
    ReLU), so each class holds identical scores."""
    rng = np.random.default_rng(seed)
    r = (rng.standard_normal((1, 1, 128)) * 128 ** -0.5).astype(np.float32)
    rk = C.idx_encode(r, "mxfp4")
    codes = np.repeat(rk.codes, n, axis=1)
    scales = np.repeat(rk.scales, n, axis=1).astype(np.int64)
    blk = np.arange(n)
    samp = (blk % 256) < 16
    scales[0, samp] += sampled_score_shift
    scales[0, ~samp] += other_shift
    assert scales.min() >= 1 and scales.max() <= 254
    return C.Idx("mxfp4", 128, codes, scales.astype(np.uint8)), samp


@pytest.mark.parametrize("bf16_scores", [False, True])
def test_sampled_select_hands_over_when_too_few_candidates(lib, bf16_scores):
    """The sample tiles score 16 times higher than every other block: the
    sampled threshold lands on the sample scores, fewer than k blocks reach
    it, and the rows go through the full-score path: the k' - |sample| extra
    ids are the lowest-indexed of the tied rest."""
    cap, Q, k, m = 20000, 8, 2048, 4
    keys, samp = _planted_keys(cap, 2, -2, 41)
    rng = _rng(41)
    q = (rng.standard_normal((1, Q, 16, 128)) * 128 ** -0.5).astype(np.float32)
    w = rng.random((1, Q, 16)).astype(np.float32)
    pos = (4 * cap - 1 - np.arange(Q)[::-1] * 4).reshape(1, Q).astype(np.int64)
    qb = C.bf16_encode(q)
    qd = C.bf16_decode(qb).astype(np.float32)
    print(f"sampled select: too few candidates, bf16={bf16_scores}", flush=True)
    call = lib.v4attn_index_topk_bf16 if bf16_scores else lib.v4attn_index_topk
    topk = call(P.dev(qb.view(np.int16)).view(torch.bfloat16), P.dev(w), P.idx_to_dev(keys),
                P.dev(pos), m, k)
    torch.cuda.synchronize()
    got = topk.cpu().numpy()
    sc = index_scores(qd, w, keys, pos, m)
    for t in range(Q):
        nv = int((pos[0, t] + 1) // m)
        s = sc[0][t]
        ids = np.arange(nv)
        assert np.sum(samp[:nv]) < k
        # expected: every sample block, then the lowest other ids (all tied)
        exp = np.sort(np.concatenate([ids[samp[:nv]], ids[~samp[:nv]][:k - int(np.sum(samp[:nv]))]]))
        assert np.all(s[samp[:nv]] > s[~samp[:nv]].max())
        assert np.array_equal(got[0, t], exp), f"query {t}"


@pytest.mark.parametrize("bf16_scores", [False, True])
def test_sampled_select_hands_over_on_ties(lib, bf16_scores):
    """All head weights zero: every score is 0, so every visible block is at
    the sampled threshold, more than the candidate list holds: the full-score
    path selects the k lowest ids."""
    cap, Q, k, m = 20000, 9, 1000, 4
    rng = _rng(43)
    y = (rng.standard_normal((1, cap, 128)) * 128 ** -0.5).astype(np.float32)
    keys = C.idx_encode(y, "mxfp4")
    q = (rng.standard_normal((1, Q, 16, 128)) * 128 ** -0.5).astype(np.float32)
    w = np.zeros((1, Q, 16), np.float32)
    pos = (4 * cap - 1 - np.arange(Q)[::-1] * 7).reshape(1, Q).astype(np.int64)
    print(f"sampled select: ties, bf16={bf16_scores}", flush=True)
    call = lib.v4attn_index_topk_bf16 if bf16_scores else lib.v4attn_index_topk
    topk = call(P.bf16_dev(q), P.dev(w), P.idx_to_dev(keys), P.dev(pos), m, k)
    torch.cuda.synchronize()
    got = topk.cpu().numpy()
    for t in range(Q):
        assert list(got[0, t]) == list(range(k)), f"query {t}"


def test_sampled_select_bf16_scores_query_tiled(lib):
    """The bf16-score ranking on the sampled path (ordinary scores: the
    selection is exact from the candidates) against the oracle's bf16
    ranking."""
    rng = _rng(47)
    Bn, Q, cap, k, m = 2, 16, 12000, 700, 4
    pos = np.empty((Bn, Q), np.int64)
    for b in range(Bn):
        pos[b] = 4 * (cap - 8) + b * 3 + np.arange(Q)
    print("sampled select: bf16 scores", flush=True)
    kinds = _index_case(lib, rng, Bn, Q, cap, 16, k, m, pos, bf16_scores=True)
    assert kinds.count("exact") >= len(kinds) // 2


def test_prefill_rows_match_single_query_calls(lib):
    """A chunk query's result does not depend on the chunk it is computed
    in: rows of a 256-query prefill call (query-tiled index scan and
    sampled selection; attention split by the per-query bound only) against
    the same queries called one at a time (Q = 1: the decode scan and the
    three-launch selector): identical top-k ids and bit-identical CSA and HCA
    outputs."""
    c, g, bits, ref = _prefill_case(8192, 256)
    k, n_win = 512, c["n_win"]
    x = _attend_inputs(lib, c, g, ref)
    qi = C.bf16_encode(g["q_idx"])
    topk = lib.v4attn_index_topk(_bf16_t(qi), P.dev(g["w"]), x["keys"], x["pos"], 4, k)
    out = lib.v4attn_csa_attend(x["q"], x["comp"], topk, x["win"], n_win, x["pos"], None, x["sc"])
    hout = lib.v4attn_hca_attend(x["q"], x["hcomp"], 128, x["hwin"], n_win, x["pos"], None, x["sc"])
    torch.cuda.synchronize()
    for t in (0, 7, 8, 131, 255):
        print(f"prefill row {t} alone", flush=True)
        one = lambda a: a[:, t:t + 1].contiguous()
        tk1 = lib.v4attn_index_topk(one(_bf16_t(qi)), one(P.dev(g["w"])), x["keys"], one(x["pos"]), 4,
                                    k)
        o1 = lib.v4attn_csa_attend(one(x["q"]), x["comp"], one(topk), x["win"], n_win, one(x["pos"]),
                                   None, x["sc"])
        h1 = lib.v4attn_hca_attend(one(x["q"]), x["hcomp"], 128, x["hwin"], n_win, one(x["pos"]),
                                   None, x["sc"])
        torch.cuda.synchronize()
        assert torch.equal(tk1[:, 0], topk[:, t]), f"row {t}: top-k ids differ"
        assert torch.equal(o1[:, 0], out[:, t]), f"row {t}: CSA output differs"
        assert torch.equal(h1[:, 0], hout[:, t]), f"row {t}: HCA output differs"
