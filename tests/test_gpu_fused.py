"""GPU parity of v4attn_csa_index_attend -- the CSA layer's indexer, top-k
selector and core attention in one call, the selector's ordering step
inside the attention kernel -- against v4attn_index_topk followed by
v4attn_csa_attend on the same inputs: identical top-k lists and bit-identical
outputs.  Cases: the decode workloads at full size (1M context, B = 4,
top-2048; 128K context, B = 8, top-1024), small ragged shapes (visible
counts below, at and just above k, rows of different lengths, several
queries per sequence, 16 to 128 heads, a sink, fp32 output), the selector's
long-tie paths at full size (a planted run resolved through the global
candidate list, one beyond the list, all head weights zero -- their chunk
lists outgrow the heads the attention loads in its first round trip, so
they also take its general list walk), and the shapes where the call runs
the two steps as they are (query-tiled scans with sampled selection, fp32
entries).  The two-call path itself is checked against the oracle by the
other GPU tests; equality carries that over."""

import numpy as np
import pytest
import torch

from oracle import codecs as C
from tests import parity as P
from tests.test_gpu_select_limits import _planted, _query
from tests.test_gpu_workloads import _decode_case

pytestmark = pytest.mark.gpu

SCALE = 512 ** -0.5


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _compare(lib, qi, w, keys, pos, m, k, q, comp, win, n_win, sink=None,
             out_dtype=torch.bfloat16):
    """Both paths on the same device inputs; asserts identical results and
    returns the fused call's (topk, out)."""
    t1 = lib.v4attn_index_topk(qi, w, keys, pos, m, k)
    o1 = lib.v4attn_csa_attend(q, comp, t1, win, n_win, pos, sink, SCALE, out_dtype=out_dtype)
    t2, o2 = lib.v4attn_csa_index_attend(qi, w, keys, m, k, q, comp, win, n_win, pos, sink, SCALE,
                                         out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(t1, t2), f"top-k differs in {int((t1 != t2).sum())} slots"
    assert torch.equal(_bits(o1), _bits(o2)), \
        f"outputs differ in {int((_bits(o1) != _bits(o2)).sum())} elements"
    return t2, o2


def _fp8_cache(rng, Bn, cap, dn=448, dr=64, tile=None):
    """An FP8 entry cache of valid codes (no NaN code): random magnitudes up
    to 8 with random signs, bf16 RoPE dims, per-entry scales near 1/16.
    With `tile`, `tile` distinct rows repeat along the cache (cheap at 1M)."""
    n = cap if tile is None else tile
    mag = rng.integers(0, 0x51, size=(Bn, n, dn), dtype=np.uint8)
    nope = mag | (rng.integers(0, 2, size=(Bn, n, dn), dtype=np.uint8) << 7)
    rope = C.bf16_encode((rng.standard_normal((Bn, n, dr)) * 0.5).astype(np.float32))
    scale = (rng.uniform(0.5, 1.5, size=(Bn, n)) / 16).astype(np.float32)
    if tile is not None:
        reps = -(-cap // tile)
        nope = np.tile(nope, (1, reps, 1))[:, :cap]
        rope = np.tile(rope, (1, reps, 1))[:, :cap]
        scale = np.tile(scale, (1, reps))[:, :cap]
    return P.kv_to_dev(C.KV("fp8", dn, dr, nope, rope, scale))


def _idx_inputs(rng, Bn, Q, cap, H_I=16, d=128):
    y = (rng.standard_normal((Bn, cap, d)) * d ** -0.5).astype(np.float32)
    keys = P.idx_to_dev(C.idx_encode(y, "mxfp4"))
    qi = P.bf16_dev((rng.standard_normal((Bn, Q, H_I, d)) * d ** -0.5).astype(np.float32))
    w = P.dev(rng.random((Bn, Q, H_I)).astype(np.float32))
    return qi, w, keys


@pytest.mark.parametrize("H,k,Q,with_sink,out_f32", [
    (64, 512, 1, False, False),
    (64, 512, 1, True, True),
    (16, 256, 3, False, False),
    (128, 1024, 2, False, False),
    (64, 2048, 1, False, False),
])
def test_fused_small_ragged(lib, H, k, Q, with_sink, out_f32):
    print(f"fused small H={H} k={k} Q={Q} sink={with_sink} f32={out_f32}", flush=True)
    rng = np.random.default_rng(H + k + Q)
    Bn, cap, n_win, m = 3, 9000, 128, 4
    qi, w, keys = _idx_inputs(rng, Bn, Q, cap)
    comp = _fp8_cache(rng, Bn, cap)
    win = _fp8_cache(rng, Bn, 256)
    q = P.bf16_dev(rng.standard_normal((Bn, Q, H, 512)).astype(np.float32))
    # per row: every block visible; just above k; below k (all selected);
    # more rows per sequence at other positions
    base = [m * cap - 1, m * (k + 37) + 3, m * (k // 2) + 1]
    pos = np.array([[base[b] - 4 * 501 * t if base[b] - 4 * 501 * t > 0 else base[b]
                     for t in range(Q)] for b in range(Bn)], np.int64)
    sink = P.dev((rng.standard_normal(H) * 2).astype(np.float32)) if with_sink else None
    _compare(lib, qi, w, keys, P.dev(pos), m, k, q, comp, win, n_win, sink,
             torch.float32 if out_f32 else torch.bfloat16)


@pytest.mark.parametrize("wid,rows", [(4, [0, 3]), (2, [0, 5])])
def test_fused_decode_full_size(lib, wid, rows):
    """The benchmark's CSA decode calls at full size: 1M context, B = 4,
    top-2048 (workload 4) and 128K context, B = 8, top-1024 (workload 2);
    16 index heads, 64 heads, a 128-token window; two rows drawn, the
    others repeat them."""
    print(f"fused CSA decode full size workload {wid}", flush=True)
    case = _decode_case(lib, wid, distinct=rows)
    c, g = case["c"], case["g"]
    qi = P.dev(case["qib"].view(np.int16)).view(torch.bfloat16)
    q = P.dev(case["qb"].view(np.int16)).view(torch.bfloat16)
    _compare(lib, qi, P.dev(g["w"]), P.idx_to_dev(case["keys"]), P.dev(g["pos"]), c["m"],
             c["k"], q, P.kv_to_dev(case["comp"]), P.kv_to_dev(case["win"]), c["n_win"])


@pytest.mark.parametrize("run,n_above", [(8000, 700), (20000, 1500)])
def test_fused_planted_ties_full_size(lib, run, n_above):
    """A run of identical scores straddling the k-th value: resolved through
    the global candidate list (8000) and by re-reading the score row
    (20000); the lower ids of the run are selected."""
    print(f"fused planted run={run} above={n_above}", flush=True)
    NV, K, M = 262144, 2048, 4
    keys, above, runs = _planted(run, n_above, 40 + run)
    qb, _, w = _query(40 + run)
    rng = np.random.default_rng(run)
    comp = _fp8_cache(rng, 1, NV, tile=4096)
    win = _fp8_cache(rng, 1, 256)
    q = P.bf16_dev(rng.standard_normal((1, 1, 64, 512)).astype(np.float32))
    pos = P.dev(np.array([[M * NV - 1]], np.int64))
    topk, _ = _compare(lib, P.dev(qb.view(np.int16)).view(torch.bfloat16), P.dev(w),
                       P.idx_to_dev(keys), pos, M, K, q, comp, win, 128)
    expect = np.sort(np.concatenate([above, runs[:K - n_above]]))
    assert np.array_equal(topk.cpu().numpy()[0, 0], expect)


def test_fused_all_zero_weights_full_size(lib):
    """w = 0: every score is 0 and the k lowest ids are the selection (two
    sequences, the second with a ragged visible count)."""
    print("fused all-zero w full size", flush=True)
    NV, K, M, Bn = 262144, 2048, 4, 2
    rng = np.random.default_rng(44)
    y = (rng.standard_normal((Bn, NV, 128)) * 128 ** -0.5).astype(np.float32)
    keys = P.idx_to_dev(C.idx_encode(y, "mxfp4"))
    qi = P.bf16_dev((rng.standard_normal((Bn, 1, 16, 128)) * 128 ** -0.5).astype(np.float32))
    w = P.dev(np.zeros((Bn, 1, 16), np.float32))
    comp = _fp8_cache(rng, Bn, NV, tile=4096)
    win = _fp8_cache(rng, Bn, 256)
    q = P.bf16_dev(rng.standard_normal((Bn, 1, 64, 512)).astype(np.float32))
    pos = P.dev(np.array([[M * NV - 1], [M * (NV - 3001) + 2]], np.int64))
    topk, _ = _compare(lib, qi, w, keys, pos, M, K, q, comp, win, 128)
    got = topk.cpu().numpy()
    for b in range(Bn):
        assert list(got[b, 0]) == list(range(K)), f"sequence {b}"


def test_fused_falls_back_to_two_steps(lib):
    """Shapes the fused step does not take: eight queries per sequence with
    16 index heads (query-tiled scan, sampled selection) and fp32 entries --
    the call runs the two steps and returns their results."""
    print("fused fallback shapes", flush=True)
    rng = np.random.default_rng(45)
    Bn, Q, cap, m, k = 1, 8, 5000, 4, 512
    qi, w, keys = _idx_inputs(rng, Bn, Q, cap)
    pos = P.dev(np.array([[m * cap - 1 - 9 * t for t in range(Q)]], np.int64))
    q = P.bf16_dev(rng.standard_normal((Bn, Q, 64, 512)).astype(np.float32))
    _compare(lib, qi, w, keys, pos, m, k, q, _fp8_cache(rng, Bn, cap), _fp8_cache(rng, Bn, 256), 128)
    # fp32 entries (D = 128), one query
    D = 128
    comp = P.kv_to_dev(C.kv_encode((rng.standard_normal((Bn, cap, D)) * 0.2).astype(np.float32),
                                   "f32", 64))
    win = P.kv_to_dev(C.kv_encode((rng.standard_normal((Bn, 256, D)) * 0.2).astype(np.float32),
                                  "f32", 64))
    qi1, w1, _ = _idx_inputs(rng, Bn, 1, cap)
    q1 = P.dev(rng.standard_normal((Bn, 1, 16, D)).astype(np.float32))
    _compare(lib, qi1, w1, keys, P.dev(np.array([[m * cap - 1]], np.int64)), m, k, q1, comp, win,
             128, out_dtype=torch.float32)


def test_launch_plan_log(lib, capfd, monkeypatch):
    """V4ATTN_LOG=1: every call prints the plan it enqueues on stderr (read
    per call); unset, nothing is printed."""
    print("launch-plan log", flush=True)
    rng = np.random.default_rng(46)
    Bn, cap, m, k = 2, 5000, 4, 512
    qi, w, keys = _idx_inputs(rng, Bn, 1, cap)
    comp, win = _fp8_cache(rng, Bn, cap), _fp8_cache(rng, Bn, 256)
    q = P.bf16_dev(rng.standard_normal((Bn, 1, 64, 512)).astype(np.float32))
    pos = P.dev(np.array([[m * cap - 1], [m * 3000 + 1]], np.int64))
    monkeypatch.setenv("V4ATTN_LOG", "1")
    capfd.readouterr()
    lib.v4attn_csa_index_attend(qi, w, keys, m, k, q, comp, win, 128, pos, None, SCALE)
    lib.v4attn_hca_attend(q, comp, m, win, 128, pos, None, SCALE)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert "v4attn: csa_index_attend: index B=2 Q=1 H_I=16" in err
    assert "path=filters, emit in the attention" in err
    assert "v4attn: csa_index_attend: attend B=2 Q=1 H=64 D=512 csa" in err
    assert "fused_select=1" in err and "loads=streaming" in err
    assert "v4attn: hca_attend B=2 Q=1 H=64 D=512 hca" in err and "loads=plain" in err
    monkeypatch.delenv("V4ATTN_LOG")
    lib.v4attn_hca_attend(q, comp, m, win, 128, pos, None, SCALE)
    torch.cuda.synchronize()
    assert "v4attn:" not in capfd.readouterr().err
