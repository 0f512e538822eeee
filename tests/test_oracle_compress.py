"""Pins of the oracle compressor: closed forms (mean pooling, one-hot gate,
identity), special cases (overlap with excluded previous slots) and a
pure-Python brute force on tiny shapes."""

import math

import numpy as np
import pytest

from oracle.compress import compress


def _rand(shape, seed, std=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * std).astype(np.float32)


@pytest.mark.parametrize("m", [1, 4, 128])
def test_uniform_gate_zero_bias_is_mean_pooling_nonoverlap(m):
    B, T, d = 2, 2 * m, 24
    kv = _rand((B, T, d), 0)
    gate = np.full((B, T, d), 0.37, dtype=np.float32)
    y = compress(kv, gate, None, None, np.zeros((m, d)), m, 0)
    ref = kv.astype(np.float64).reshape(B, T // m, m, d).mean(axis=2)
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-7)


def test_uniform_gate_zero_bias_is_mean_pooling_overlap():
    m, B, T, d = 4, 2, 16, 8
    cur, prev = _rand((B, T, d), 1), _rand((B, T, d), 2)
    gate = np.zeros((B, T, d), np.float32)
    y = compress(cur, gate, prev, gate, np.zeros((2 * m, d)), m, 0)
    c = cur.astype(np.float64).reshape(B, T // m, m, d)
    p = prev.astype(np.float64).reshape(B, T // m, m, d)
    ref = (c.sum(2) + p.sum(2)) / (2 * m)
    ref[:, 0] = c[:, 0].mean(1)            # block 0 has no previous block
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-7)
    # t0 > 0: block t0/m does see its previous rows
    y2 = compress(cur, gate, prev, gate, np.zeros((2 * m, d)), m, 8)
    ref2 = (c.sum(2) + p.sum(2)) / (2 * m)
    assert np.allclose(y2, ref2, rtol=1e-6, atol=1e-7)


def test_none_gate_and_bias_equal_zero():
    m, B, T, d = 4, 1, 8, 8
    kv = _rand((B, T, d), 3)
    a = compress(kv, None, None, None, None, m, 0)
    b = compress(kv, np.zeros_like(kv), None, None, np.zeros((m, d)), m, 0)
    assert np.array_equal(a, b)


def test_one_hot_gate_selects_token():
    m, B, T, d = 4, 1, 8, 6
    kv = _rand((B, T, d), 4)
    gate = np.zeros((B, T, d), np.float32)
    gate[0, 2] = 80.0          # block 0, slot 2
    gate[0, 7] = 80.0          # block 1, slot 3
    y = compress(kv, gate, None, None, None, m, 0)
    assert np.allclose(y[0, 0], kv[0, 2], rtol=1e-6)
    assert np.allclose(y[0, 1], kv[0, 7], rtol=1e-6)


def test_bias_per_slot_and_channel_shifts_weights():
    # a bias of +80 on slot j of channel c selects token j for that channel only
    m, d = 4, 5
    kv = _rand((1, m, d), 5)
    bias = np.zeros((m, d), np.float32)
    bias[1, 0] = 80.0
    bias[3, 4] = 80.0
    y = compress(kv, np.zeros_like(kv), None, None, bias, m, 0)
    assert np.isclose(y[0, 0, 0], kv[0, 1, 0], rtol=1e-6)
    assert np.isclose(y[0, 0, 4], kv[0, 3, 4], rtol=1e-6)
    assert np.allclose(y[0, 0, 1:4], kv[0, :, 1:4].astype(np.float64).mean(0), rtol=1e-6)


def test_m1_is_identity():
    kv = _rand((2, 7, 9), 6)
    y = compress(kv, _rand((2, 7, 9), 7), None, None, _rand((1, 9), 8), 1, 0)
    assert np.array_equal(y, kv.astype(np.float64))


def test_overlap_with_excluded_prev_equals_nonoverlap():
    m, B, T, d = 4, 2, 12, 8
    cur, prev = _rand((B, T, d), 9), _rand((B, T, d), 10)
    gc, gp = _rand((B, T, d), 11), np.full((B, T, d), -1e4, np.float32)
    bias = _rand((2 * m, d), 12, 0.5)
    y = compress(cur, gc, prev, gp, bias, m, 4)
    y0 = compress(cur, gc, None, None, bias[m:], m, 4)
    assert np.allclose(y, y0, rtol=1e-12, atol=0)


def test_streaming_chunks_equal_one_call():
    # compressing [0, T) at once equals [0, T1) then [T1, T) with the prev
    # rows of the second call starting at token T1 - m
    m, B, T, T1, d = 4, 1, 24, 8, 8
    a_cur, a_prev = _rand((B, T, d), 13), _rand((B, T, d), 14)
    g_cur, g_prev = _rand((B, T, d), 15), _rand((B, T, d), 16)
    bias = _rand((2 * m, d), 17, 0.5)
    # prev-role rows of a call at t0 are tokens t0-m .. : build token-indexed
    # prev streams and slice them per call
    tok_prev = np.concatenate([np.zeros((B, m, d), np.float32), a_prev], 1)   # token t -> row t+m
    tok_gp = np.concatenate([np.zeros((B, m, d), np.float32), g_prev], 1)
    full = compress(a_cur, g_cur, tok_prev[:, 0:T], tok_gp[:, 0:T], bias, m, 0)
    p1 = compress(a_cur[:, :T1], g_cur[:, :T1], tok_prev[:, 0:T1], tok_gp[:, 0:T1], bias, m, 0)
    p2 = compress(a_cur[:, T1:], g_cur[:, T1:], tok_prev[:, T1:T], tok_gp[:, T1:T], bias, m, T1)
    assert np.array_equal(full, np.concatenate([p1, p2], 1))


def _brute(kv_cur, gate_cur, kv_prev, gate_prev, bias, m, t0):
    B, T, d = kv_cur.shape
    out = np.zeros((B, T // m, d))
    for b in range(B):
        for j in range(T // m):
            for c in range(d):
                terms = []
                if kv_prev is not None and not (t0 == 0 and j == 0):
                    for u in range(m):
                        terms.append((float(gate_prev[b, m * j + u, c]) + float(bias[u, c]),
                                      float(kv_prev[b, m * j + u, c])))
                off = m if kv_prev is not None else 0
                for u in range(m):
                    terms.append((float(gate_cur[b, m * j + u, c]) + float(bias[off + u, c]),
                                  float(kv_cur[b, m * j + u, c])))
                mx = max(t[0] for t in terms)
                den = sum(math.exp(z - mx) for z, _ in terms)
                out[b, j, c] = sum(math.exp(z - mx) * v for z, v in terms) / den
    return out


@pytest.mark.parametrize("overlap,t0", [(False, 0), (True, 0), (True, 8)])
def test_bruteforce_tiny(overlap, t0):
    m, B, T, d = 4, 2, 12, 5
    cur, gc = _rand((B, T, d), 20), _rand((B, T, d), 21)
    prev = _rand((B, T, d), 22) if overlap else None
    gp = _rand((B, T, d), 23) if overlap else None
    bias = _rand(((2 if overlap else 1) * m, d), 24, 0.5)
    y = compress(cur, gc, prev, gp, bias, m, t0)
    ref = _brute(cur, gc, prev, gp, bias, m, t0)
    assert np.allclose(y, ref, rtol=2e-7, atol=1e-9)   # oracle rounds to fp32
