"""Pins of the oracle core attention: reductions to textbook attention (torch
scaled_dot_product_attention in float64 on the CPU), CSA-with-everything equal
to HCA, window-only equal to sliding-window attention, sink limits and
closed forms, permutation invariance."""

import math

import numpy as np
import pytest
import torch

from oracle import codecs as C
from oracle.attend import csa_attend, hca_attend


def _f32(shape, seed, std=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * std).astype(np.float32)


def _kv_f32(x, d_nope):
    return C.kv_encode(x, "f32", d_nope)


def _sdpa(q, k, v, mask, scale):
    """torch's textbook attention in float64; q [H][D], k,v [n][D], mask [n]."""
    qt = torch.from_numpy(q)[None, :, None, :]          # [1][H][1][D]
    kt = torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(v)[None, None].expand(1, q.shape[0], -1, -1)
    mt = torch.from_numpy(mask)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    return o[0, :, 0, :].numpy()


def test_m1_no_window_is_causal_softmax_attention():
    # HCA with m = 1 over raw tokens and no window = textbook causal attention
    T, H, D = 37, 3, 16
    toks = _f32((1, T, D), 0, 0.5)
    comp = _kv_f32(toks, 8)
    win = _kv_f32(np.zeros((1, 4, D), np.float32), 8)
    q = _f32((1, T, H, D), 1)
    pos = np.arange(T)[None, :]
    _, out = hca_attend(q, "f32", comp, 1, win, 0, pos, None, 0.3, "f32")
    k = toks[0].astype(np.float64)
    for t in range(T):
        mask = np.arange(T) <= t
        ref = _sdpa(q[0, t].astype(np.float64), k, k, mask, 0.3)
        assert np.allclose(out[0, t], ref, rtol=1e-12, atol=1e-14)


def test_window_only_is_sliding_window_attention():
    T, H, D, n_win, R = 50, 2, 8, 7, 16
    toks = _f32((1, T, D), 2)
    q = _f32((1, T, H, D), 3)
    comp = _kv_f32(_f32((1, 10, D), 4), 4)
    k = toks[0].astype(np.float64)
    for t in range(T):
        ring = np.zeros((1, R, D), np.float32)
        for u in range(max(0, t - R + 1), t + 1):
            ring[0, u % R] = toks[0, u]
        win = _kv_f32(ring, 4)
        topk = np.full((1, 1, 3), -1)
        _, out = csa_attend(q[:, t:t + 1], "f32", comp, topk, win, n_win,
                            np.array([[t]]), None, 0.5, "f32")
        mask = (np.arange(T) <= t) & (np.arange(T) > t - n_win)
        ref = _sdpa(q[0, t].astype(np.float64), k, k, mask, 0.5)
        assert np.allclose(out[0, 0], ref, rtol=1e-12, atol=1e-14)


def test_csa_with_all_blocks_equals_hca():
    m, n, H, D, R = 4, 25, 4, 16, 8
    comp = C.kv_encode(_f32((2, n, D), 5, 0.3), "fp8", 12)
    win = C.kv_encode(_f32((2, R, D), 6, 0.3), "fp8", 12)
    q = C.bf16_encode(_f32((2, 3, H, D), 7))
    pos = np.array([[50, 77, 99], [3, 40, 60]])
    _, hca = hca_attend(q, "bf16", comp, m, win, 5, pos, None, 0.25, "bf16")
    topk = np.full((2, 3, 40), -1)
    for b in range(2):
        for t in range(3):
            nv = min((pos[b, t] + 1) // m, n)
            topk[b, t, :nv] = np.arange(nv)
    _, csa = csa_attend(q, "bf16", comp, topk, win, 5, pos, None, 0.25, "bf16")
    assert np.array_equal(hca, csa)


def test_permutation_invariance_of_selected_set():
    comp = _kv_f32(_f32((1, 30, 8), 8), 4)
    win = _kv_f32(_f32((1, 8, 8), 9), 4)
    q = _f32((1, 1, 2, 8), 10)
    ids = np.array([[[3, 17, 4, 29, 0, -1]]])
    perm = np.array([[[-1, 29, 0, 17, 4, 3]]])
    _, a = csa_attend(q, "f32", comp, ids, win, 4, np.array([[200]]), None, 1.0, "f32")
    _, b = csa_attend(q, "f32", comp, perm, win, 4, np.array([[200]]), None, 1.0, "f32")
    assert np.allclose(a, b, rtol=1e-14, atol=0)


def test_sink_limits_and_closed_form():
    D, H = 8, 3
    comp = _kv_f32(_f32((1, 5, D), 11), 4)
    win = _kv_f32(np.zeros((1, 1, D), np.float32), 4)
    q = _f32((1, 1, H, D), 12)
    ids = np.array([[[0, 1, 2, 3, 4]]])
    pos = np.array([[100]])
    _, none = csa_attend(q, "f32", comp, ids, win, 0, pos, None, 0.7, "f32")
    _, low = csa_attend(q, "f32", comp, ids, win, 0, pos, np.full(H, -1e4), 0.7, "f32")
    _, high = csa_attend(q, "f32", comp, ids, win, 0, pos, np.full(H, 1e4), 0.7, "f32")
    assert np.allclose(none, low, rtol=1e-14, atol=0)
    assert np.max(np.abs(high)) < 1e-300
    # one entry and a sink z: out = v * e^l / (e^l + e^z)
    one = np.array([[[2, -1, -1, -1, -1]]])
    z = np.array([0.3, -1.0, 2.0])
    _, o = csa_attend(q, "f32", comp, one, win, 0, pos, z, 0.7, "f32")
    v = comp.nope[0, 2].astype(np.float64).tolist() + comp.rope[0, 2].astype(np.float64).tolist()
    for h in range(H):
        l = 0.7 * sum(float(q[0, 0, h, c]) * v[c] for c in range(D))
        wgt = math.exp(l) / (math.exp(l) + math.exp(z[h]))
        assert np.allclose(o[0, 0, h], np.array(v) * wgt, rtol=1e-12)


def test_empty_set_gives_zero_output():
    comp = _kv_f32(_f32((1, 5, 8), 13), 4)
    win = _kv_f32(_f32((1, 4, 8), 14), 4)
    q = _f32((1, 2, 2, 8), 15)
    ids = np.full((1, 2, 3), -1)
    bits, out = csa_attend(q, "f32", comp, ids, win, 0, np.array([[5, 6]]), None, 1.0, "f32")
    assert np.all(out == 0)
    _, out2 = hca_attend(q, "f32", comp, 4, win, 4, np.array([[-1, -5]]), None, 1.0, "f32")
    assert np.all(out2 == 0)


def test_fp8_entries_attend_as_their_decoded_values():
    # HCA over FP8 entries = textbook attention over the float64 decoded entries
    m, n, H, D, R, n_win = 4, 12, 2, 16, 8, 6
    comp8 = C.kv_encode(_f32((1, n, D), 16, 0.2), "fp8", 12)
    win = C.kv_encode(_f32((1, R, D), 17, 0.2), "fp8", 12)
    qb = C.bf16_encode(_f32((1, 2, H, D), 18))
    pos = np.array([[40, 45]])
    _, out = hca_attend(qb, "bf16", comp8, m, win, n_win, pos, None, 0.5, "f32")
    q = C.bf16_decode(qb)
    for t in range(2):
        p = pos[0, t]
        nv = min((p + 1) // m, n)
        ent = np.concatenate([C.kv_decode_rows(comp8, 0, np.arange(nv)),
                              C.kv_decode_rows(win, 0, np.arange(p - n_win + 1, p + 1) % R)])
        ref = _sdpa(q[0, t], ent, ent, np.ones(len(ent), bool), 0.5)
        assert np.allclose(out[0, t], ref, rtol=1e-12, atol=1e-15)


def test_window_and_compressed_share_one_softmax_without_dedup():
    # duplicating an entry in both sets doubles its weight (no de-duplication)
    D = 4
    v0 = np.array([[[1.0, 0, 0, 0]]], np.float32)
    comp = _kv_f32(np.concatenate([v0, np.array([[[0, 1.0, 0, 0]]], np.float32)], 1), 2)
    win = _kv_f32(v0, 2)                               # ring of 1: token p at row 0
    q = np.zeros((1, 1, 1, D), np.float32)             # all logits 0
    ids = np.array([[[0, 1]]])
    _, out = csa_attend(q, "f32", comp, ids, win, 1, np.array([[9]]), None, 1.0, "f32")
    assert np.allclose(out[0, 0, 0], [2 / 3, 1 / 3, 0, 0], rtol=1e-14)
