"""Pins of the paged-cache and decode-append oracle ([Notes §11] KV cache
table): hand-computed row maps, the identity and permuted tables against the
contiguous cache, and the incremental compressor against the one-shot
definition of the same stream."""

import numpy as np
import pytest

from oracle import codecs as C
from oracle.compress import compress
from oracle.paged import append_entry, entries_per_page, logical_view, pool_rows


def test_entries_per_page():
    # a 512-token page: 128 CSA entries (m = 4), 4 HCA entries (m = 128)
    assert entries_per_page(512, 4) == 128
    assert entries_per_page(512, 128) == 4
    assert entries_per_page(2048, 1) == 2048
    with pytest.raises(AssertionError):
        entries_per_page(96, 4)                # not a multiple of lcm(4, 128)


def test_pool_rows_hand_example():
    # pages [3, 1] of 4 entries: logical 0..3 -> pool 12..15, 4..7 -> 4..7
    assert pool_rows([3, 1], 4, [0, 3, 4, 7]).tolist() == [12, 15, 4, 7]
    assert pool_rows([0, 5, 2], 2, [5, 4, 2]).tolist() == [5, 4, 10]


def _cache(B, n, seed):
    rng = np.random.default_rng(seed)
    y = rng.normal(size=(B, n, 512)).astype(np.float32)
    return C.kv_encode(y, "fp8", 448), C.idx_encode(rng.normal(size=(B, n, 128)), "mxfp4")


def _to_pool(a, perm, P):
    """Place page j of sequence b of a [B][n_pg * P][...] array at pool page perm[b][j]."""
    B, n_pg = perm.shape
    out = np.zeros((1, (perm.max() + 1) * P) + a.shape[2:], a.dtype)
    for b in range(B):
        for j in range(n_pg):
            out[0, perm[b, j] * P:(perm[b, j] + 1) * P] = a[b, j * P:(j + 1) * P]
    return out


@pytest.mark.parametrize("permute", [False, True])
def test_logical_view_restores_the_cache(permute):
    B, n_pg, P = 3, 4, 8
    kv, ix = _cache(B, n_pg * P, 7)
    perm = np.arange(B * n_pg).reshape(B, n_pg)
    if permute:
        perm = np.random.default_rng(3).permutation(B * n_pg + 5)[:B * n_pg].reshape(B, n_pg)
    pool_kv = C.KV("fp8", 448, 64, _to_pool(kv.nope, perm, P), _to_pool(kv.rope, perm, P),
                   _to_pool(kv.scale, perm, P))
    pool_ix = C.Idx("mxfp4", 128, _to_pool(ix.codes, perm, P), _to_pool(ix.scales, perm, P))
    lv, li = logical_view(pool_kv, perm, P), logical_view(pool_ix, perm, P)
    for got, want in ((lv.nope, kv.nope), (lv.rope, kv.rope), (lv.scale, kv.scale),
                      (li.codes, ix.codes), (li.scales, ix.scales)):
        assert got.shape == want.shape and np.array_equal(got, want)
    if not permute:
        # the identity table: sequence b is the pool's b-th run of n_pg pages
        assert np.array_equal(lv.nope, pool_kv.nope[0].reshape(B, n_pg * P, 448))


def test_append_hand_case():
    # m = 2, zero gates and bias: each entry is the mean of its two tokens;
    # odd positions complete a block, even ones do not
    kv = np.array([[1.0, -2.0], [3.0, 4.0], [5.0, 0.5], [7.0, 1.5]])
    st = {"kv_cur": kv, "gate_cur": None}
    assert append_entry(st, 0, 2, None) is None
    assert np.allclose(append_entry(st, 1, 2, None), [2.0, 1.0])
    assert append_entry(st, 2, 2, None) is None
    assert np.allclose(append_entry(st, 3, 2, None), [6.0, 1.0])


@pytest.mark.parametrize("m,overlap", [(4, True), (4, False), (16, False), (1, False)])
def test_append_matches_one_shot_compress(m, overlap):
    rng = np.random.default_rng(m + overlap)
    T, d = 12 * m, 40
    st = {"kv_cur": rng.normal(size=(T, d)).astype(np.float32),
          "gate_cur": rng.normal(size=(T, d)).astype(np.float32)}
    if overlap:
        st["kv_prev"] = rng.normal(size=(T, d)).astype(np.float32)
        st["gate_prev"] = rng.normal(size=(T, d)).astype(np.float32)
    slots = 2 * m if overlap else m
    bias = rng.normal(size=(slots, d)).astype(np.float32) * 0.5
    # the one-shot call: previous-role rows of tokens t0 - m .. t0 + T - m - 1
    prev = gate_prev = None
    if overlap:
        prev = np.concatenate([np.zeros((m, d), np.float32), st["kv_prev"][:T - m]])[None]
        gate_prev = np.concatenate([np.zeros((m, d), np.float32), st["gate_prev"][:T - m]])[None]
    want = compress(st["kv_cur"][None], st["gate_cur"][None], prev, gate_prev, bias, m, 0)[0]
    got = [append_entry(st, p, m, bias) for p in range(T)]
    done = [p for p in range(T) if got[p] is not None]
    assert done == [i * m + m - 1 for i in range(T // m)]
    assert np.array_equal(np.stack([got[p] for p in done]), want)
