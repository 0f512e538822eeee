"""Pins of the oracle indexer and selector: exact rational recomputation of
the FP4 scores, one-hot / zero head weights, brute-force selection, visibility."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codecs as C
from oracle.indexer import index_scores, index_topk, n_visible, topk_from_scores


def _keys_mx(n, d, seed):
    y = (np.random.default_rng(seed).standard_normal((1, n, d)) / np.sqrt(d)).astype(np.float32)
    return C.idx_encode(y, "mxfp4"), y


def _e2m1_twice(nib):
    # 2 * e2m1 value as an integer, from the OCP table (0,1,2,3,4,6,8,12 halves)
    mag = [0, 1, 2, 3, 4, 6, 8, 12][nib & 7]
    return -mag if nib & 8 else mag


def _exact_mx_vector(packed, scales):
    """Exact rational values of one MXFP4 vector."""
    vals = []
    for i, byte in enumerate(packed):
        for nib in (byte & 0xF, byte >> 4):
            g = len(vals) // 32
            vals.append(Fraction(_e2m1_twice(int(nib)), 2) * Fraction(2) ** (int(scales[g]) - 127))
    return vals


def test_fp4_scores_exact_rational():
    d, n, H = 64, 9, 3
    keys, _ = _keys_mx(n, d, 0)
    rng = np.random.default_rng(1)
    q = (rng.standard_normal((1, 1, H, d)) / 8).astype(np.float32)
    w = rng.random((1, 1, H)).astype(np.float32)
    pos = np.array([[4 * n - 1]])
    s = index_scores(q, w, keys, pos, 4)[0][0]
    qp, qs = C.mxfp4_encode(q[0, 0])
    for j in range(n):
        kv = _exact_mx_vector(keys.codes[0, j], keys.scales[0, j])
        tot = Fraction(0)
        for h in range(H):
            qv = _exact_mx_vector(qp[h], qs[h])
            dot = sum(a * b for a, b in zip(qv, kv))
            tot += Fraction(float(w[0, 0, h])) * max(dot, Fraction(0))
        assert s[j] == pytest.approx(float(tot), rel=1e-15, abs=1e-300)


def test_f32_scores_are_plain_relu_dots():
    d, n, H = 16, 7, 2
    rng = np.random.default_rng(2)
    K = rng.standard_normal((1, n, d)).astype(np.float32)
    keys = C.idx_encode(K, "f32")
    q = rng.standard_normal((1, 1, H, d)).astype(np.float32)
    w = rng.random((1, 1, H)).astype(np.float32)
    s = index_scores(q, w, keys, np.array([[100]]), 4)[0][0]
    for j in range(n):
        ref = sum(float(w[0, 0, h]) * max(0.0, sum(float(q[0, 0, h, c]) * float(K[0, j, c])
                                                   for c in range(d))) for h in range(H))
        assert s[j] == pytest.approx(ref, rel=1e-12)


def test_one_hot_w_gives_relu_of_head_dot():
    d, n, H = 128, 20, 4
    keys, _ = _keys_mx(n, d, 3)
    q = (np.random.default_rng(4).standard_normal((1, 1, H, d)) / 11).astype(np.float32)
    Kd = C.mxfp4_decode(keys.codes[0], keys.scales[0])
    qd = C.mxfp4_decode(*C.mxfp4_encode(q[0, 0]))
    for h in range(H):
        w = np.zeros((1, 1, H), np.float32)
        w[0, 0, h] = 1.0
        s = index_scores(q, w, keys, np.array([[10 ** 6]]), 4)[0][0]
        assert np.array_equal(s, np.maximum(Kd @ qd[h], 0))


def test_zero_w_selects_lowest_indices():
    keys, _ = _keys_mx(40, 64, 5)
    q = np.ones((1, 1, 2, 64), np.float32)
    w = np.zeros((1, 1, 2), np.float32)
    topk, _ = index_topk(q, w, keys, np.array([[159]]), 4, 7)
    assert list(topk[0, 0]) == list(range(7))


def test_visibility():
    assert n_visible(-1, 4, 100) == 0
    assert n_visible(2, 4, 100) == 0
    assert n_visible(3, 4, 100) == 1
    assert n_visible(4095, 4, 2000) == 1024
    assert n_visible(4095, 4, 1000) == 1000
    assert n_visible(1048575, 128, 8192) == 8192
    assert n_visible(126, 128, 8192) == 0 and n_visible(127, 128, 8192) == 1


def test_topk_bruteforce_with_planted_ties():
    rng = np.random.default_rng(6)
    for trial in range(30):
        n = int(rng.integers(1, 200))
        s = rng.integers(0, 12, n).astype(np.float64) * 0.5   # many exact ties
        k = int(rng.integers(1, 260))
        got = topk_from_scores(s, k)
        # brute force: repeatedly take the max, lowest index on ties
        left = list(range(n))
        chosen = []
        for _ in range(min(k, n)):
            best = max(left, key=lambda i: (s[i], -i))
            chosen.append(best)
            left.remove(best)
        assert list(got[:min(k, n)]) == sorted(chosen)
        assert all(v == -1 for v in got[min(k, n):])


def test_k_at_least_nvis_selects_all():
    keys, _ = _keys_mx(30, 64, 7)
    q = np.ones((1, 1, 2, 64), np.float32)
    w = np.ones((1, 1, 2), np.float32)
    topk, sc = index_topk(q, w, keys, np.array([[4 * 12 + 1]]), 4, 20)   # n_vis = 12
    assert list(topk[0, 0]) == list(range(12)) + [-1] * 8
    assert len(sc[0][0]) == 12


# ---------------------------------------------------------------- BF16-score selector
# [Notes §9]: the selector's index scores cut from FP32 to BF16.

def test_bf16_selector_hand_computed_ties():
    # 1.0, 1 + 2^-10, 1 + 2^-9 all round to bf16 1.0 (the bf16 step at 1 is
    # 2^-7), so the fp32 ranking {1, 2} becomes a three-way tie: ids 0, 1 win
    s = np.array([1.0, 1.0 + 2.0 ** -10, 1.0 + 2.0 ** -9, 0.5])
    assert list(topk_from_scores(s, 2, "f32")) == [1, 2]
    assert list(topk_from_scores(s, 2, "bf16")) == [0, 1]


def test_bf16_selector_round_half_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 (even mantissa) and 1 + 2^-7:
    # ties to even -> 1.0, equal to id 1; 1 + 3 * 2^-8 is halfway between
    # 1 + 2^-7 (odd mantissa) and 1 + 2^-6 (even): rounds up, above id 3
    s = np.array([1.0 + 2.0 ** -8, 1.0, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -7])
    # bf16 values: [1.0, 1.0, 1 + 2^-6, 1 + 2^-7] -> order 2, 3, 0, 1
    assert list(topk_from_scores(s, 1, "bf16")) == [2]
    assert list(topk_from_scores(s, 2, "bf16")) == [2, 3]
    assert list(topk_from_scores(s, 3, "bf16")) == [0, 2, 3]
    # fp32 order: 2, 3, 0, 1 as well, but id 0 beats id 1 by value there
    assert list(topk_from_scores(s, 3, "f32")) == [0, 2, 3]
    s2 = np.array([1.0, 1.0 + 2.0 ** -8])          # bf16: equal -> lower id
    assert list(topk_from_scores(s2, 1, "f32")) == [1]
    assert list(topk_from_scores(s2, 1, "bf16")) == [0]


def test_bf16_selector_is_fp32_on_bf16_values():
    # scores already representable in bf16 rank identically in both modes
    rng = np.random.default_rng(9)
    for _ in range(20):
        n = int(rng.integers(1, 300))
        bits = rng.integers(0x3C00, 0x4400, n).astype(np.uint16)   # positive bf16 values
        s = C.bf16_decode(bits)
        k = int(rng.integers(1, 320))
        assert np.array_equal(topk_from_scores(s, k, "bf16"), topk_from_scores(s, k, "f32"))


def test_bf16_selector_order_property():
    # every selected id's bf16 value >= every other's; at the boundary value
    # the selected ids are the lowest ones
    rng = np.random.default_rng(10)
    for _ in range(20):
        n = int(rng.integers(2, 400))
        s = rng.normal(1.0, 0.01, n)
        k = int(rng.integers(1, n))
        sel = topk_from_scores(s, k, "bf16")
        sel = sel[sel >= 0]
        v = C.bf16_decode(C.bf16_encode(C.f32(s)))
        rest = np.setdiff1d(np.arange(n), sel)
        assert v[sel].min() >= v[rest].max()
        t = v[sel].min()
        tie_sel = sel[v[sel] == t]
        tie_rest = rest[v[rest] == t]
        assert len(tie_rest) == 0 or tie_sel.max() < tie_rest.min()
