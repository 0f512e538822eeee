"""GPU parity of the top-k selector on the paths that only long ties reach,
at the 1M-context decode shape (262144 visible blocks, top-2048, 16 index
heads, one query per sequence -- the headline decode scan).

The exact threshold search works on the ids that share the k-th score's top
19 key bits.  Up to 4096 of them are resolved in LDS; up to 16384 through the
query's global candidate list; beyond that the search re-reads the whole
score row.  The cases below force each of the two larger paths with planted
runs of identical keys (identical keys give bit-identical scores on both
sides), and the all-equal case (every head weight 0) at full size, where the
lower-block-id rule of the selector decides every id.

Keys are built from one random MXFP4 key r: a block whose key is r with
every e8m0 scale byte raised by j scores exactly 2^j times r's score (FP4
products with power-of-two scales are exact and ReLU is positively
homogeneous), so the expected selection is known in closed form and is
checked both against that form and against the oracle."""

import numpy as np
import pytest
import torch

from oracle import codecs as C
from oracle.indexer import index_scores, topk_from_scores
from tests import parity as P

pytestmark = pytest.mark.gpu

NV, K, H, D, M = 262144, 2048, 16, 128, 4


def _planted(run, n_above, seed):
    """Keys of one sequence: n_above ids score 2 or 4 times s_r, `run` ids
    score s_r, the rest s_r / 2, / 4 or / 32.  Returns (keys, above ids,
    run ids ascending)."""
    rng = np.random.default_rng(seed)
    r = (rng.standard_normal((1, 1, D)) * D ** -0.5).astype(np.float32)
    rk = C.idx_encode(r, "mxfp4")
    codes = np.repeat(rk.codes, NV, axis=1)
    scales = np.repeat(rk.scales, NV, axis=1).astype(np.int64)
    perm = rng.permutation(NV)
    above = np.sort(perm[:n_above])
    runs = np.sort(perm[n_above:n_above + run])
    rest = perm[n_above + run:]
    scales[0, above] += rng.choice([1, 2], size=n_above)[:, None]
    scales[0, rest] += rng.choice([-1, -2, -5], size=len(rest))[:, None]
    assert scales.min() >= 1 and scales.max() <= 254
    keys = C.Idx("mxfp4", D, codes, scales.astype(np.uint8))
    return keys, above, runs


def _query(seed):
    rng = np.random.default_rng(seed + 1)
    q = (rng.standard_normal((1, 1, H, D)) * D ** -0.5).astype(np.float32)
    w = rng.random((1, 1, H)).astype(np.float32)
    qb = C.bf16_encode(q)
    return qb, C.bf16_decode(qb).astype(np.float32), w


def _run_case(lib, run, n_above, seed, bf16_scores):
    keys, above, runs = _planted(run, n_above, seed)
    qb, qd, w = _query(seed)
    pos = np.array([[M * NV - 1]], np.int64)
    sc = index_scores(qd, w, keys, pos, M)[0][0]
    s_r = sc[runs[0]]
    assert s_r > 0 and np.all(sc[runs] == s_r), "planted run must score identically"
    assert np.all(sc[above] >= 2 * s_r) and np.sum(sc < s_r) == NV - run - n_above
    expect = np.sort(np.concatenate([above, runs[:K - n_above]]))
    dtype = "bf16" if bf16_scores else "f32"
    assert np.array_equal(topk_from_scores(sc, K, dtype), expect)
    call = lib.v4attn_index_topk_bf16 if bf16_scores else lib.v4attn_index_topk
    print(f"select run={run} above={n_above} scores={dtype}", flush=True)
    topk = call(P.dev(qb.view(np.int16)).view(torch.bfloat16), P.dev(w), P.idx_to_dev(keys),
                P.dev(pos), M, K)
    torch.cuda.synchronize()
    got = topk.cpu().numpy()[0, 0]
    assert np.array_equal(got, expect), \
        f"{int(np.sum(got != expect))} ids differ from the lower-id selection"


@pytest.mark.parametrize("bf16_scores", [False, True])
def test_select_run_beyond_candidate_list(lib, bf16_scores):
    # 20000 ids at the k-th value: more than the 16384 candidate slots
    _run_case(lib, 20000, 1500, 31, bf16_scores)


def test_select_run_in_global_candidate_list(lib):
    # about 8000 ids at the k-th value: more than LDS holds, within the list
    _run_case(lib, 8000, 700, 32, False)


@pytest.mark.parametrize("bf16_scores", [False, True])
def test_select_all_zero_weights_full_size(lib, bf16_scores):
    # w = 0: all 262144 scores are 0, the k lowest ids win; two sequences,
    # the second with a ragged visible count
    rng = np.random.default_rng(33)
    Bn = 2
    y = (rng.standard_normal((Bn, NV, D)) * D ** -0.5).astype(np.float32)
    keys = C.idx_encode(y, "mxfp4")
    q = (rng.standard_normal((Bn, 1, H, D)) * D ** -0.5).astype(np.float32)
    w = np.zeros((Bn, 1, H), np.float32)
    pos = np.array([[M * NV - 1], [M * (NV - 3001) + 2]], np.int64)
    call = lib.v4attn_index_topk_bf16 if bf16_scores else lib.v4attn_index_topk
    print(f"select all-zero w full size bf16={bf16_scores}", flush=True)
    topk = call(P.bf16_dev(q), P.dev(w), P.idx_to_dev(keys), P.dev(pos), M, K)
    torch.cuda.synchronize()
    got = topk.cpu().numpy()
    for b in range(Bn):
        assert list(got[b, 0]) == list(range(K)), f"sequence {b}"
