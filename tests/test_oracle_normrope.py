"""Pins of the query / KV-entry RMSNorm and partial RoPE oracle ([Notes §9])
against closed forms and invariants."""

import math

import numpy as np

from oracle import codecs as C
from oracle.attend import hca_attend
from oracle.compress import compress
from oracle.normrope import default_inv_freq, entry_positions, rms_norm, rope, rope_angles


def test_rms_norm_closed_forms():
    # [3, 4] with eps 0.5: mean square 12.5, + 0.5 = 13
    assert np.allclose(rms_norm([3.0, 4.0], [1.0, 1.0], 0.5), [3 / math.sqrt(13), 4 / math.sqrt(13)])
    # a constant vector normalises to +-1, then scales by gamma
    g = np.arange(1, 9, dtype=np.float64)
    assert np.allclose(rms_norm(np.full(8, -2.5), g, 0.0), -g)
    # unit weight, no eps: mean square 1
    x = np.random.default_rng(1).normal(size=(5, 512)) * 7
    y = rms_norm(x, np.ones(512), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0)


def test_rope_hand_computed_pair():
    # one rotated pair, inverse frequency 0.5, position 1: angle 0.5
    x = np.array([9.0, 1.0, 0.0])
    y = rope(x, 1, np.array([0.5], np.float32))
    assert y[0] == 9.0                                   # unrotated dim untouched
    assert np.allclose(y[1:], [math.cos(0.5), math.sin(0.5)])


def test_rope_pairs_are_adjacent_dims():
    # e_0 of the rotated part moves within dims (0, 1), e_2 within (2, 3)
    inv = np.array([1.0, 0.25], np.float32)
    e0 = rope(np.array([1.0, 0.0, 0.0, 0.0]), 3, inv)
    e2 = rope(np.array([0.0, 0.0, 1.0, 0.0]), 3, inv)
    assert np.allclose(e0, [math.cos(3.0), math.sin(3.0), 0, 0])
    assert np.allclose(e2, [0, 0, math.cos(0.75), math.sin(0.75)])


def test_rope_preserves_pair_norms_and_inverts():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(7, 512))
    pos = rng.integers(0, 1 << 20, size=7)
    inv = default_inv_freq(64)
    y = rope(x, pos, inv)
    assert np.array_equal(y[:, :448], x[:, :448])
    n0 = x[:, 448::2] ** 2 + x[:, 449::2] ** 2
    n1 = y[:, 448::2] ** 2 + y[:, 449::2] ** 2
    assert np.allclose(n0, n1)
    assert np.allclose(rope(y, pos, inv, sign=-1), x)


def test_rope_relative_positions():
    # with power-of-two frequencies and small positions the fp32 angles are
    # exact, so the rotated dot depends on the position difference only
    inv = np.array([1.0, 0.5, 0.25, 0.125], np.float32)
    rng = np.random.default_rng(3)
    q, k = rng.normal(size=8), rng.normal(size=8)
    d1 = rope(q, 17, inv) @ rope(k, 5, inv)
    d2 = rope(q, 112, inv) @ rope(k, 100, inv)
    assert abs(d1 - d2) < 1e-12


def test_rope_angle_is_the_fp32_product():
    inv = np.array([0.1], np.float32)
    p = (1 << 20) + 1
    a = rope_angles(p, inv)[0]
    assert a == float(np.float32(np.float32(p) * np.float32(0.1)))
    assert a != p * 0.1                                  # not the exact product


def test_default_table_and_entry_positions():
    inv = default_inv_freq(64)
    assert inv[0] == 1.0 and len(inv) == 32
    assert np.isclose(inv[1], 10000 ** (-2 / 64))
    assert list(entry_positions([0, 1, 5], 4)) == [3, 7, 23]
    assert list(entry_positions([0, 9], 1)) == [0, 9]


def test_compress_with_norm_rope_composes():
    # the compressor's nr output is RMSNorm then RoPE of its plain output at
    # the blocks' last-token positions
    rng = np.random.default_rng(4)
    B, T, d, m, t0 = 1, 16, 128, 4, 8
    kv, z = rng.normal(size=(B, T, d)), rng.normal(size=(B, T, d))
    nr = dict(gamma=rng.uniform(0.5, 1.5, d), eps=1e-6, inv_freq=default_inv_freq(64))
    plain = compress(kv, z, None, None, None, m, t0)
    got = compress(kv, z, None, None, None, m, t0, nr=nr)
    pos = np.array([11, 15, 19, 23])
    want = C.f32(rope(rms_norm(plain, nr["gamma"], nr["eps"]), pos[None, :], nr["inv_freq"]))
    assert np.array_equal(got, want.astype(np.float64))


def test_output_rotation_undoes_the_entry_rotation():
    # one visible entry (window only, at the query's own position): attention
    # weight 1, so the output is the stored (rotated) entry rotated back by the
    # query position = the unrotated entry (RoPE dims) exactly up to rounding
    rng = np.random.default_rng(5)
    D, H, p = 512, 2, 300
    inv = default_inv_freq(64)
    v = rng.normal(size=D) / math.sqrt(D)
    v_rot = rope(v, p, inv)
    win = C.kv_encode(v_rot[None, None, :].repeat(1, axis=1), "fp8", 448)
    comp = C.kv_encode(np.zeros((1, 1, D)), "fp8", 448)
    q = C.bf16_encode(rng.normal(size=(1, 1, H, D)).astype(np.float32))
    nr = dict(gamma=np.ones(D), eps=1e-6, inv_freq=inv)
    # ring of one row holds token p (p mod 1 = 0); n_win = 1
    _, out = hca_attend(q, "bf16", comp, 1 << 30, win, 1, np.array([[p]]), None, 0.05, "f32", nr=nr)
    stored = C.kv_decode_rows(win, 0, np.array([0]))[0]
    want = rope(stored, p, inv, sign=-1)
    for h in range(H):
        assert np.allclose(out[0, 0, h], want, atol=1e-12)
    # the RoPE dims come back to the unrotated entry up to the bf16 storage
    assert np.allclose(out[0, 0, 0, 448:], v[448:], atol=2e-2 * np.abs(v[448:]).max())


def test_partial_options_switch_single_steps_off():
    # gamma None: RoPE alone (norms of the rotated pairs kept); inv_freq None:
    # RMSNorm alone (mean square 1 with unit weights); both: the identity
    from oracle.normrope import norm_rope
    x = np.random.default_rng(5).normal(size=(3, 512)) * 4
    inv = default_inv_freq(64)
    only_rope = norm_rope(x, np.array([7, 8, 9]), dict(gamma=None, eps=0.0, inv_freq=inv))
    assert np.array_equal(only_rope[:, :448], x[:, :448])
    pair = lambda a: np.hypot(a[:, 448::2], a[:, 449::2])
    assert np.allclose(pair(only_rope), pair(x))
    assert not np.allclose(only_rope[:, 448:], x[:, 448:])
    only_norm = norm_rope(x, np.array([7, 8, 9]), dict(gamma=np.ones(512), eps=0.0, inv_freq=None))
    assert np.allclose(np.mean(only_norm ** 2, axis=-1), 1.0)
    assert np.allclose(only_norm * np.sqrt(np.mean(x ** 2, axis=-1, keepdims=True)), x)
    none = norm_rope(x, 0, dict(gamma=None, eps=0.0, inv_freq=None))
    assert np.array_equal(none, x)
