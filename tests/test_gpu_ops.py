"""GPU parity of each C-ABI call against the CPU oracle on identical input
bytes, at sizes that span several tiles / splits with ragged tails, plus edge
cases (empty sets, k >= n_vis, ties, sinks, window-only, negative positions)."""

import numpy as np
import pytest
import torch

from long_context_attention_v4attn_amd import synth
from oracle import codecs as C
from oracle.attend import csa_attend, hca_attend
from oracle.compress import compress
from oracle.indexer import index_scores, index_topk
from tests import parity as P

pytestmark = pytest.mark.gpu


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


# ---------------------------------------------------------------- compress

@pytest.mark.parametrize("m,overlap,t0,fmt,in_bf16", [
    (32, True, 0, "fp8", True),
    (64, True, 128, "f32", False),
    (128, False, 0, "f32", True),
    (4, True, 0, "fp8", False),
    (4, True, 64, "fp8", True),
    (128, False, 0, "fp8", False),
    (128, False, 256, "fp8", True),
    (1, False, 5, "fp8", False),
    (4, False, 0, "f32", False),
    (4, True, 8, "f32", False),
])
def test_compress_kv(lib, m, overlap, t0, fmt, in_bf16):
    print(f"compress kv m={m} overlap={overlap} t0={t0} fmt={fmt} bf16={in_bf16}", flush=True)
    rng = _rng(m * 7 + t0)
    Bn, d, dn = 2, 512, 448
    T = 3 * m if m > 1 else 37
    g = synth.compress_inputs(3, Bn, T, d, m, overlap, t0)
    if in_bf16:   # inputs rounded to bf16 on both sides
        for k in ("kv_cur", "gate_cur", "kv_prev", "gate_prev"):
            if g[k] is not None:
                g[k] = C.bf16_decode(C.bf16_encode(g[k])).astype(np.float32)
    y = compress(g["kv_cur"], g["gate_cur"], g["kv_prev"], g["gate_prev"], g["bias"], m, t0)
    cap = (t0 + T) // m + 3
    out = lib.KVCache.empty(Bn, cap, dn, d - dn, lib.KV_FP8_BF16ROPE if fmt == "fp8" else lib.F32)
    up = P.bf16_dev if in_bf16 else P.dev
    lib.v4attn_compress(up(g["kv_cur"]), up(g["gate_cur"]),
                        None if g["kv_prev"] is None else up(g["kv_prev"]),
                        None if g["gate_prev"] is None else up(g["gate_prev"]),
                        P.dev(g["bias"]), m, t0, out)
    torch.cuda.synchronize()
    back = P.kv_from_dev(out)
    r0, r1 = t0 // m, t0 // m + T // m
    if fmt == "fp8":
        sub = C.KV("fp8", dn, d - dn, back.nope[:, r0:r1], back.rope[:, r0:r1], back.scale[:, r0:r1])
        P.check_fp8_rows(sub, y, dn)
        assert np.all(back.nope[:, :r0] == 0) and np.all(back.nope[:, r1:] == 0), "rows outside the call written"
    else:
        full = np.concatenate([back.nope, back.rope], -1)[:, r0:r1]
        P.check_f32_rows(full, y)


@pytest.mark.parametrize("fmt,overlap,d,m", [("mxfp4", True, 128, 4), ("mxfp4", False, 128, 4),
                                             ("f32", True, 64, 4), ("mxfp4", True, 256, 4),
                                             ("mxfp4", False, 128, 128), ("mxfp4", True, 128, 32)])
def test_compress_index_keys(lib, fmt, overlap, d, m):
    print(f"compress keys fmt={fmt} overlap={overlap} d={d} m={m}", flush=True)
    Bn, T, t0 = 3, 16 * m, 4 * m
    g = synth.compress_inputs(2, Bn, T, d, m, overlap, t0)
    y = compress(g["kv_cur"], g["gate_cur"], g["kv_prev"], g["gate_prev"], g["bias"], m, t0)
    cap = (t0 + T) // m + 4
    out = lib.IdxCache.empty(Bn, cap, d, lib.IDX_MXFP4 if fmt == "mxfp4" else lib.F32)
    lib.v4attn_compress(P.dev(g["kv_cur"]), P.dev(g["gate_cur"]),
                        None if g["kv_prev"] is None else P.dev(g["kv_prev"]),
                        None if g["gate_prev"] is None else P.dev(g["gate_prev"]),
                        P.dev(g["bias"]), m, t0, out)
    torch.cuda.synchronize()
    back = P.idx_from_dev(out)
    r0, r1 = t0 // m, (t0 + T) // m
    if fmt == "mxfp4":
        P.check_mxfp4_rows(C.Idx("mxfp4", d, back.codes[:, r0:r1], back.scales[:, r0:r1]), y)
    else:
        P.check_f32_rows(back.codes[:, r0:r1], y)


def test_compress_ring_wraps(lib):
    # m = 1 stores token rows at (t0 + j) mod cap
    rng = _rng(11)
    x = _f32(rng, (1, 6, 512), 0.05)
    out = lib.KVCache.empty(1, 4, 448, 64, lib.KV_FP8_BF16ROPE)
    lib.v4attn_compress(P.dev(x), None, None, None, None, 1, 10, out)
    torch.cuda.synchronize()
    back = P.kv_from_dev(out)
    ref = C.kv_encode(x, "fp8", 448)
    for j in range(6):
        r = (10 + j) % 4
        if j >= 2:   # rows of the last 4 tokens survive
            assert np.array_equal(C.e4m3_decode(back.nope[0, r]), C.e4m3_decode(ref.nope[0, j]))
            assert back.scale[0, r] == ref.scale[0, j]


# ---------------------------------------------------------------- index + top-k

def _index_case(lib, rng, Bn, Q, cap, H, k, m, pos, key_fmt="mxfp4", d=128, w=None, keys=None,
                bf16_scores=False):
    if keys is None:
        y = _f32(rng, (Bn, cap, d), d ** -0.5)
        keys = C.idx_encode(y, key_fmt)
    q = _f32(rng, (Bn, Q, H, d), d ** -0.5)
    if w is None:
        w = rng.random((Bn, Q, H)).astype(np.float32)
    qb = C.bf16_encode(q)
    qd = C.bf16_decode(qb).astype(np.float32)
    call = lib.v4attn_index_topk_bf16 if bf16_scores else lib.v4attn_index_topk
    topk = call(P.dev(qb.view(np.int16)).view(torch.bfloat16), P.dev(w), P.idx_to_dev(keys),
                P.dev(pos), m, k)
    torch.cuda.synchronize()
    sc = index_scores(qd, w, keys, pos, m)
    g = topk.cpu().numpy()
    check = P.check_topk_row_bf16 if bf16_scores else P.check_topk_row
    kinds = []
    for b in range(Bn):
        for t in range(Q):
            kinds.append(check(g[b, t], sc[b][t], k))
    return kinds


@pytest.mark.parametrize("cap,k,H", [(1000, 64, 16), (5003, 300, 16), (3000, 100, 64), (777, 1024, 32)])
def test_index_topk_mxfp4(lib, cap, k, H):
    print(f"index mxfp4 cap={cap} k={k} H={H}", flush=True)
    rng = _rng(cap + k)
    Bn, Q, m = 2, 3, 4
    pos = np.array([[4 * cap - 1, 4 * (cap // 2) + 2, 37], [4 * cap + 100, 4 * cap - 5, 3]], np.int64)
    kinds = _index_case(lib, rng, Bn, Q, cap, H, k, m, pos)
    assert kinds.count("exact") >= len(kinds) // 2


@pytest.mark.parametrize("cap,k,H", [(1000, 64, 16), (5003, 300, 16), (3000, 100, 64), (777, 1024, 32)])
def test_index_topk_bf16_scores(lib, cap, k, H):
    # the BF16-score selector: the oracle's bf16 ranking (ties to the lower id)
    print(f"index bf16 scores cap={cap} k={k} H={H}", flush=True)
    rng = _rng(cap + k)
    Bn, Q, m = 2, 3, 4
    pos = np.array([[4 * cap - 1, 4 * (cap // 2) + 2, 37], [4 * cap + 100, 4 * cap - 5, 3]], np.int64)
    kinds = _index_case(lib, rng, Bn, Q, cap, H, k, m, pos, bf16_scores=True)
    assert kinds.count("exact") >= len(kinds) // 2


def test_index_topk_bf16_scores_f32_keys_and_ties(lib):
    print("index bf16 scores: f32 keys; all-equal scores", flush=True)
    rng = _rng(11)
    _index_case(lib, rng, 1, 1, 1024, 4, 64, 4, np.array([[4095]], np.int64), key_fmt="f32", d=64,
                bf16_scores=True)
    # all-zero head weights: every score is 0, the k lowest ids win
    Bn, Q, cap, H, k = 1, 2, 3000, 16, 50
    pos = np.array([[4 * cap - 1, 4 * 1000 - 1]], np.int64)
    w = np.zeros((Bn, Q, H), np.float32)
    keys = C.idx_encode(_f32(rng, (Bn, cap, 128), 0.1), "mxfp4")
    q = _f32(rng, (Bn, Q, H, 128), 0.1)
    topk = lib.v4attn_index_topk_bf16(P.dev(q), P.dev(w), P.idx_to_dev(keys), P.dev(pos), 4, k)
    g = topk.cpu().numpy()
    assert list(g[0, 0]) == list(range(k)) and list(g[0, 1]) == list(range(k))


def test_index_topk_f32_workload1_shape(lib):
    rng = _rng(5)
    pos = np.array([[4095]], np.int64)
    _index_case(lib, rng, 1, 1, 1024, 4, 64, 4, pos, key_fmt="f32", d=64)


def test_index_topk_ties_lower_index_wins(lib):
    # all-zero head weights: every score is 0, the k lowest ids win
    rng = _rng(6)
    Bn, Q, cap, H, k = 1, 2, 3000, 16, 50
    pos = np.array([[4 * cap - 1, 4 * 1000 - 1]], np.int64)
    w = np.zeros((Bn, Q, H), np.float32)
    y = _f32(rng, (Bn, cap, 128), 0.1)
    keys = C.idx_encode(y, "mxfp4")
    q = _f32(rng, (Bn, Q, H, 128), 0.1)
    topk = lib.v4attn_index_topk(P.dev(q), P.dev(w), P.idx_to_dev(keys), P.dev(pos), 4, k)
    g = topk.cpu().numpy()
    assert list(g[0, 0]) == list(range(k)) and list(g[0, 1]) == list(range(k))
    # planted duplicate keys: identical blocks score identically; lower id first
    keys.codes[0, 10:20] = keys.codes[0, 500]
    keys.scales[0, 10:20] = keys.scales[0, 500]
    w1 = rng.random((Bn, Q, H)).astype(np.float32)
    topk = lib.v4attn_index_topk(P.dev(q), P.dev(w1), P.idx_to_dev(keys), P.dev(pos), 4, 5)
    sc = index_scores(q, w1, keys, pos, 4)
    g = topk.cpu().numpy()
    for t in range(Q):
        P.check_topk_row(g[0, t], sc[0][t], 5)


@pytest.mark.parametrize("Q,kind", [(3, "nonpositive"), (3, "mixed"), (16, "nonpositive"), (16, "mixed")])
def test_index_topk_signed_weights(lib, Q, kind):
    """Head weights of any sign (w is any real): "nonpositive" -- w < 0 and
    one query direction for all heads, so about half the blocks score
    exactly 0 (every ReLU term zero, the products -0) and the rest below 0:
    the top k are the k lowest ids among the zeros, with -0 ranked equal to
    +0; "mixed" -- weights of both signs, scores of both signs.  Q = 3 takes
    the decode scan and the three-launch selector, Q = 16 the query-tiled
    scan with the sampled-threshold selection."""
    print(f"index signed weights Q={Q} {kind}", flush=True)
    rng = _rng(97 + Q + len(kind))
    Bn, cap, H, k, m, d = 1, 5000, 16, 300, 4, 128
    y = _f32(rng, (Bn, cap, d), d ** -0.5)
    keys = C.idx_encode(y, "mxfp4")
    if kind == "nonpositive":
        q1 = _f32(rng, (Bn, Q, 1, d), d ** -0.5)
        q = np.repeat(q1, H, axis=2)
        w = -(rng.random((Bn, Q, H)).astype(np.float32) + 0.1)
    else:
        q = _f32(rng, (Bn, Q, H, d), d ** -0.5)
        w = rng.standard_normal((Bn, Q, H)).astype(np.float32)
    pos = np.full((Bn, Q), m * cap - 1, np.int64)
    pos[0, 1] = m * (cap // 3) + 1
    qb = C.bf16_encode(q)
    qd = C.bf16_decode(qb).astype(np.float32)
    topk = lib.v4attn_index_topk(P.dev(qb.view(np.int16)).view(torch.bfloat16), P.dev(w),
                                 P.idx_to_dev(keys), P.dev(pos), m, k)
    torch.cuda.synchronize()
    sc = index_scores(qd, w, keys, pos, m)
    g = topk.cpu().numpy()
    for t in range(Q):
        s = sc[0][t]
        if kind == "nonpositive":
            assert np.all(s <= 0) and np.sum(s == 0) > k, "the planted zero scores"
            expect = np.nonzero(s == 0)[0][:k]
            assert np.array_equal(g[0, t], expect), f"query {t}: not the k lowest ids of the zeros"
        else:
            assert (s > 0).any() and (s < 0).any()
            P.check_topk_row(g[0, t], s, k)


def test_index_topk_small_and_empty_visibility(lib):
    rng = _rng(7)
    cap, k = 64, 16
    pos = np.array([[-1, 2, 3, 40, 63, 255, 10 ** 6]], np.int64)   # n_vis 0,0,1,10,16,64,64
    _index_case(lib, rng, 1, pos.shape[1], cap, 16, k, 4, pos)


# ---------------------------------------------------------------- attend

def _attend_inputs(rng, Bn, Q, H, n_comp, R, fmt="fp8", dn=448, dr=64):
    D = dn + dr
    comp = C.kv_encode(_f32(rng, (Bn, n_comp, D), D ** -0.5 * 3), fmt, dn)
    win = C.kv_encode(_f32(rng, (Bn, R, D), D ** -0.5 * 3), fmt, dn)
    q = _f32(rng, (Bn, Q, H, D), 1.0)
    return comp, win, q


def _run_attend(lib, kind, q, q_bf16, comp, win, n_win, pos, sink, scale, topk=None, m=None,
                out_dtype=torch.bfloat16):
    qd = P.bf16_dev(q) if q_bf16 else P.dev(q)
    sk = None if sink is None else P.dev(sink.astype(np.float32))
    if kind == "csa":
        o = lib.v4attn_csa_attend(qd, P.kv_to_dev(comp), P.dev(topk.astype(np.int32)),
                                  P.kv_to_dev(win), n_win, P.dev(pos), sk, scale,
                                  out_dtype=out_dtype)
    else:
        o = lib.v4attn_hca_attend(qd, P.kv_to_dev(comp), m, P.kv_to_dev(win), n_win,
                                  P.dev(pos), sk, scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("H,n_comp,m,with_sink", [(64, 300, 4, False), (16, 1000, 4, True),
                                                   (128, 90, 1, False), (48, 2100, 128, False)])
def test_hca_attend_fp8(lib, H, n_comp, m, with_sink):
    print(f"hca fp8 H={H} n_comp={n_comp} m={m} sink={with_sink}", flush=True)
    rng = _rng(H + n_comp)
    Bn, Q, R, n_win = 2, 2, 160, 128
    comp, win, q = _attend_inputs(rng, Bn, Q, H, n_comp, R)
    pos = np.array([[m * n_comp + 5, m * (n_comp // 3) + 1], [40, m * n_comp - 1]], np.int64)
    sink = rng.standard_normal(H) if with_sink else None
    qb = C.bf16_encode(q)
    scale = 512 ** -0.5
    _, ref = hca_attend(qb, "bf16", comp, m, win, n_win, pos, sink, scale, "bf16")
    o = _run_attend(lib, "hca", q, True, comp, win, n_win, pos, sink, scale, m=m)
    P.check_out(o, ref)


@pytest.mark.parametrize("H,k,n_comp", [(64, 64, 500), (64, 333, 2000), (32, 1024, 900)])
def test_csa_attend_fp8(lib, H, k, n_comp):
    print(f"csa fp8 H={H} k={k} n_comp={n_comp}", flush=True)
    rng = _rng(H * 3 + k)
    Bn, Q, R, n_win = 2, 3, 256, 128
    comp, win, q = _attend_inputs(rng, Bn, Q, H, n_comp, R)
    pos = np.array([[4 * n_comp - 1, 1000, 60], [4 * n_comp + 7, 200, 0]], np.int64)
    topk = np.full((Bn, Q, k), -1, np.int64)
    for b in range(Bn):
        for t in range(Q):
            nv = min((pos[b, t] + 1) // 4, n_comp)
            kk = min(k, nv)
            topk[b, t, :kk] = np.sort(rng.choice(nv, kk, replace=False)) if kk else []
    topk[0, 0, 3] = -1          # holes and out-of-range ids are skipped
    topk[1, 0, 5] = n_comp + 9
    qb = C.bf16_encode(q)
    scale = 512 ** -0.5
    _, ref = csa_attend(qb, "bf16", comp, topk, win, n_win, pos, None, scale, "bf16")
    o = _run_attend(lib, "csa", q, True, comp, win, n_win, pos, None, scale, topk=topk)
    P.check_out(o, ref)
    o32 = _run_attend(lib, "csa", q, True, comp, win, n_win, pos, None, scale, topk=topk,
                      out_dtype=torch.float32)
    P.check_out(o32, ref)


@pytest.mark.parametrize("kind", ["hca", "csa"])
def test_attend_fp8_error_within_operand_rounding_bound(lib, kind):
    """The FP8 path's arithmetic: probabilities enter the PV product as bf16
    MFMA operands and each split's normalised partial O/l is stored in bf16;
    everything else is fp32 on exactly widened entries.  Per output element
    (h, d) that bounds the error by 2^-9 (A + 2 M): A = sum_e P_e |v_e,d|
    (probability rounding), M = max_e |v_e,d| (a partial and the output are
    means of the v_e,d, each rounded once).  Checked on fp32 outputs against
    the oracle's exact float64 result, on lists long enough for many splits."""
    from oracle.attend import window_positions
    print(f"{kind} fp8 operand-rounding bound", flush=True)
    rng = _rng(41 if kind == "hca" else 42)
    Bn, Q, H, R, n_win, m = 2, 1, 64, 160, 128, 4
    n_comp = 8000 if kind == "hca" else 3000
    comp, win, q = _attend_inputs(rng, Bn, Q, H, n_comp, R)
    pos = np.array([[m * n_comp - 1], [m * 5000 + 2]], np.int64)
    scale = 512 ** -0.5
    qb = C.bf16_encode(q)
    if kind == "hca":
        _, ref = hca_attend(qb, "bf16", comp, m, win, n_win, pos, None, scale, "f32")
        o = _run_attend(lib, "hca", q, True, comp, win, n_win, pos, None, scale, m=m,
                        out_dtype=torch.float32)
        ids = [np.arange(min((p + 1) // m, n_comp)) for p in pos[:, 0]]
    else:
        k = 1024
        ids = [np.sort(rng.choice(min((p + 1) // m, n_comp), k, replace=False)) for p in pos[:, 0]]
        topk = np.stack(ids)[:, None, :]
        _, ref = csa_attend(qb, "bf16", comp, topk, win, n_win, pos, None, scale, "f32")
        o = _run_attend(lib, "csa", q, True, comp, win, n_win, pos, None, scale, topk=topk,
                        out_dtype=torch.float32)
    g = o.cpu().numpy().astype(np.float64)
    qd = C.bf16_decode(qb).astype(np.float64)
    worst = 0.0
    for b in range(Bn):
        p = int(pos[b, 0])
        V = np.concatenate([C.kv_decode_rows(comp, b, ids[b]),
                            C.kv_decode_rows(win, b, window_positions(p, n_win) % R)])
        s = scale * (qd[b, 0] @ V.T)
        Pm = np.exp(s - s.max(axis=1, keepdims=True))
        Pm /= Pm.sum(axis=1, keepdims=True)
        A = Pm @ np.abs(V)                       # [H][D]
        M = np.abs(V).max(axis=0)[None, :]
        bound = 2.0 ** -9 * (A + 2 * M) * 1.01 + 1e-7
        err = np.abs(g[b, 0] - ref[b, 0])
        worst = max(worst, float((err / bound).max()))
    assert worst <= 1.0, f"error reaches {worst:.3f} of the operand-rounding bound"


def test_attend_fp8_edge_cases(lib):
    rng = _rng(21)
    Bn, Q, H, n_comp, R = 1, 4, 16, 50, 130
    comp, win, q = _attend_inputs(rng, Bn, Q, H, n_comp, R)
    qb = C.bf16_encode(q)
    scale = 0.1
    # window-only (k slots all empty) and an empty set (no window, no entries)
    topk = np.full((Bn, Q, 8), -1, np.int64)
    pos = np.array([[0, 5, 129, 1000]], np.int64)
    for n_win in (128, 1, 0):
        _, ref = csa_attend(qb, "bf16", comp, topk, win, n_win, pos, None, scale, "bf16")
        o = _run_attend(lib, "csa", q, True, comp, win, n_win, pos, None, scale, topk=topk)
        P.check_out(o, ref)
    # sink that dominates: output -> ~0 relative to the entries
    sink = np.full(H, 30.0)
    _, ref = hca_attend(qb, "bf16", comp, 4, win, 16, pos, sink, scale, "bf16")
    o = _run_attend(lib, "hca", q, True, comp, win, 16, pos, sink, scale, m=4)
    P.check_out(o, ref)
    # negative positions see nothing
    pos_neg = np.array([[-1, -7, 3, 3]], np.int64)
    _, ref = hca_attend(qb, "bf16", comp, 4, win, 16, pos_neg, None, scale, "bf16")
    o = _run_attend(lib, "hca", q, True, comp, win, 16, pos_neg, None, scale, m=4)
    P.check_out(o, ref)


@pytest.mark.parametrize("kind,H", [("hca", 64), ("hca", 32), ("csa", 64)])
def test_attend_fp8_running_max_jumps(lib, kind, H):
    """Entries whose logits jump by ~9.5 (base-2) units part-way through a
    split: the running max moves after the split's first tile, so the rare
    rescale step runs (joint tile max, P rewritten, accumulators and
    denominators scaled) -- and the planted entries carry about half of the
    softmax mass, so a wrong rescale factor shows.  Two jumps sit in
    different splits, so the merge combines splits of different maxima."""
    print(f"attend running-max jumps {kind} H={H}", flush=True)
    rng = _rng(401 + H + len(kind))
    Bn, Q, R, n_win, D = 1, 2, 160, 128, 512
    n_comp = 2048 if kind == "csa" else 3000
    scale = D ** -0.5
    rows = _f32(rng, (Bn, n_comp, D), D ** -0.5 * 0.5)
    base = _f32(rng, (Bn, 1, 1, D), 1.0)
    q = base + _f32(rng, (Bn, Q, H, D), 0.02)
    u = base[0, 0, 0] / float(base[0, 0, 0] @ base[0, 0, 0])
    hot = [100, 101, 1000, 1001]
    for e in hot:                      # logit ln(750) ~ 6.6 nats above the rest
        rows[0, e] = np.log(750.0) / scale * u
    comp = C.kv_encode(rows, "fp8", 448)
    win = C.kv_encode(_f32(rng, (Bn, R, D), D ** -0.5 * 0.5), "fp8", 448)
    qb = C.bf16_encode(q)
    pos = np.array([[n_comp * (4 if kind == "csa" else 1) + 40, n_comp * (4 if kind == "csa" else 1) - 1]],
                   np.int64)
    if kind == "csa":
        topk = np.broadcast_to(np.arange(n_comp, dtype=np.int64), (Bn, Q, n_comp)).copy()
        _, ref = csa_attend(qb, "bf16", comp, topk, win, n_win, pos, None, scale, "bf16")
        o = _run_attend(lib, "csa", q, True, comp, win, n_win, pos, None, scale, topk=topk)
    else:
        _, ref = hca_attend(qb, "bf16", comp, 1, win, n_win, pos, None, scale, "bf16")
        o = _run_attend(lib, "hca", q, True, comp, win, n_win, pos, None, scale, m=1)
    P.check_out(o, ref)


@pytest.mark.parametrize("H,n_comp,m,n_win,with_sink,f32_out", [
    (64, 30, 1, 16, True, False),      # one split: the kernel writes the output itself
    (64, 3000, 1, 128, False, True),   # 17 splits of 6 tiles, fp32 output
    (128, 700, 4, 128, True, False),   # two groups of 64 heads
    (64, 9000, 1, 128, False, False),  # 16 splits of 18 tiles
])
def test_hca_attend_64_head_groups(lib, H, n_comp, m, n_win, with_sink, f32_out):
    """HCA lists at H % 64 == 0 (the 64-head workgroups): rows whose splits
    hold every tile count from full down to none (positions spread over the
    list), a window-only row, an empty row (negative position), a sink."""
    print(f"hca 64-head groups H={H} n_comp={n_comp} m={m} n_win={n_win}", flush=True)
    rng = _rng(H + n_comp + n_win)
    Bn, Q, R = 2, 4, 160
    comp, win, q = _attend_inputs(rng, Bn, Q, H, n_comp, R)
    last = m * n_comp - 1
    pos = np.array([[last, m * (n_comp // 2) + 3, m * 33 + 1, m - 2],
                    [last + 77, m * (n_comp // 7), 5, -3]], np.int64)
    sink = rng.standard_normal(H) if with_sink else None
    qb = C.bf16_encode(q)
    scale = 512 ** -0.5
    _, ref = hca_attend(qb, "bf16", comp, m, win, n_win, pos, sink, scale, "bf16")
    o = _run_attend(lib, "hca", q, True, comp, win, n_win, pos, sink, scale, m=m,
                    out_dtype=torch.float32 if f32_out else torch.bfloat16)
    P.check_out(o, ref)


@pytest.mark.parametrize("kind,q_bf16", [("csa", False), ("hca", True)])
def test_attend_f32_entries(lib, kind, q_bf16):
    rng = _rng(31)
    Bn, Q, H, n_comp, R, n_win, dn, dr = 2, 2, 8, 1024, 128, 128, 64, 64
    comp, win, q = _attend_inputs(rng, Bn, Q, H, n_comp, R, fmt="f32", dn=dn, dr=dr)
    pos = np.array([[4095, 1000], [4095, 77]], np.int64)
    scale = 128 ** -0.5
    qin = C.bf16_encode(q) if q_bf16 else q
    if kind == "csa":
        topk = np.full((Bn, Q, 64), -1, np.int64)
        for b in range(Bn):
            for t in range(Q):
                nv = min((pos[b, t] + 1) // 4, n_comp)
                kk = min(64, nv)
                topk[b, t, :kk] = np.sort(rng.choice(nv, kk, replace=False))
        _, ref = csa_attend(qin, "bf16" if q_bf16 else "f32", comp, topk, win, n_win, pos, None,
                            scale, "f32")
        o = _run_attend(lib, "csa", q, q_bf16, comp, win, n_win, pos, None, scale, topk=topk,
                        out_dtype=torch.float32)
    else:
        _, ref = hca_attend(qin, "bf16" if q_bf16 else "f32", comp, 4, win, n_win, pos, None,
                            scale, "f32")
        o = _run_attend(lib, "hca", q, q_bf16, comp, win, n_win, pos, None, scale, m=4,
                        out_dtype=torch.float32)
    P.check_out(o, ref, tol=1e-4)
