"""The allocation-free index call (v4attn_index_topk_noalloc) against the
workspace call (v4attn_index_topk) through the C ABI: bit-equal top-k ids on
two calls in a row, the second smaller than the first (the fixed scratch
keeps the first call's contents), on both scan paths (query-tiled prefill
scan with its prep kernel; one-query decode scan that clears its own
counters); and the host-side rejection of a call beyond the fixed scratch."""

import numpy as np
import pytest
import torch

from oracle import codecs as C
from oracle.indexer import index_scores
from tests import parity as P

pytestmark = pytest.mark.gpu


def _inputs(seed, Bn, Q, cap, H=16, d=128, m=4):
    rng = np.random.default_rng(seed)
    keys = C.idx_encode((rng.standard_normal((Bn, cap, d)) * d ** -0.5).astype(np.float32), "mxfp4")
    q = (rng.standard_normal((Bn, Q, H, d)) * d ** -0.5).astype(np.float32)
    w = rng.random((Bn, Q, H)).astype(np.float32)
    hi = m * cap + 50
    pos = rng.integers(hi // 2, hi, size=(Bn, Q)).astype(np.int64)
    pos[0, 0] = m * cap - 1
    return keys, q, w, pos


def _both(lib, keys, q, w, pos, m, k):
    qd, wd, kd, pd = P.bf16_dev(q), P.dev(w), P.idx_to_dev(keys), P.dev(pos)
    Bn, Q = pos.shape
    ref = lib.v4attn_index_topk(qd, wd, kd, pd, m, k)
    got = torch.full((Bn, Q, k), -7, dtype=torch.int32, device="cuda")
    lib.v4attn_index_topk_noalloc(qd, wd, kd, pd, m, k, got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def test_noalloc_matches_workspace_call_twice(lib):
    m = 4
    # 1: query-tiled scan (16 queries per sequence), 2 sequences x 40000 blocks
    keys, q, w, pos = _inputs(71, 2, 16, 40000)
    print("noalloc call 1: B=2 Q=16 cap=40000 k=1024", flush=True)
    got, ref = _both(lib, keys, q, w, pos, m, 1024)
    assert np.array_equal(got, ref)
    sc = index_scores(C.bf16_decode(C.bf16_encode(q)).astype(np.float32), w, keys, pos, m)
    for t in (0, 5, 15):
        P.check_topk_row(got[1, t], sc[1][t], 1024)
    # 2: smaller, one-query decode scan (its own counter clearing): 3 x 9000
    keys, q, w, pos = _inputs(72, 3, 1, 9000)
    print("noalloc call 2: B=3 Q=1 cap=9000 k=256", flush=True)
    got, ref = _both(lib, keys, q, w, pos, m, 256)
    assert np.array_equal(got, ref)
    sc = index_scores(C.bf16_decode(C.bf16_encode(q)).astype(np.float32), w, keys, pos, m)
    for b in range(3):
        P.check_topk_row(got[b, 0], sc[b][0], 256)


def test_noalloc_rejects_beyond_fixed_scratch(lib):
    # 28 one-query rows over 262144 blocks need more than the 32 MiB array:
    # refused on the host before anything is enqueued (the inputs are never read)
    Bn, cap = 28, 262144
    keys = lib.IdxCache.empty(Bn, cap, 128, lib.IDX_MXFP4)
    q = torch.zeros(Bn, 1, 16, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(Bn, 1, 16, dtype=torch.float32, device="cuda")
    pos = torch.zeros(Bn, 1, dtype=torch.int64, device="cuda")
    topk = torch.empty(Bn, 1, 2048, dtype=torch.int32, device="cuda")
    with pytest.raises(lib.V4AttnError, match="fixed 32 MiB"):
        lib.v4attn_index_topk_noalloc(q, w, keys, pos, 4, 2048, topk)
