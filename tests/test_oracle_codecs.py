"""Pins of the oracle's number formats against the OCP definitions, torch's
library casts and brute-force nearest-value search (independent of the
oracle's binade-based encoders)."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import codecs as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_finite_e4m3():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    return codes, C.e4m3_decode(codes)


def test_e4m3_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = C.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert nan.sum() == 2  # only S.1111.111


def test_e4m3_golden_codes():
    with open(os.path.join(GOLDEN, "ocp_fp8_e4m3.json")) as f:
        g = json.load(f)
    for item in g["codes"]:
        assert C.e4m3_decode(np.uint8(item["code"])) == item["value"], item
        if item["value"] != 0:
            assert C.e4m3_encode(item["value"]) == item["code"], item


def test_e4m3_encode_matches_torch_dense_sweep():
    rng = np.random.default_rng(0)
    codes, vals = _all_finite_e4m3()
    pos = np.unique(vals[vals > 0])
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
        mids, -mids, pos, -pos,
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64),
        np.nextafter(mids.astype(np.float32), np.float32(-np.inf)).astype(np.float64),
    ])
    x = x.astype(np.float32).astype(np.float64)
    ours = C.e4m3_encode(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # compare decoded values (+0 and -0 are the same value)
    assert np.array_equal(C.e4m3_decode(ours), C.e4m3_decode(ref))


def test_e4m3_encode_is_nearest_with_even_ties_bruteforce():
    rng = np.random.default_rng(1)
    codes, vals = _all_finite_e4m3()
    x = np.concatenate([rng.uniform(-460, 460, 3000),
                        rng.standard_normal(3000) * 2.0 ** -8])
    x = x.astype(np.float32).astype(np.float64)
    enc = C.e4m3_encode(x)
    for xi, ci in zip(x, enc):
        xs = min(max(xi, -448.0), 448.0)
        d = np.abs(vals - xs)
        best = d.min()
        cands = [int(c) for c, dv in zip(codes, d) if dv == best]
        if len(cands) > 1:  # tie: even mantissa (LSB of the code) wins; +-0 both fine
            cands = [c for c in cands if c & 1 == 0] or cands
        assert C.e4m3_decode(ci) in [C.e4m3_decode(c) for c in cands], (xi, ci, cands)


def test_e4m3_saturates_and_never_nan():
    x = np.array([448.0, 449.0, 464.0, 1e6, -1e6, -470.0])
    enc = C.e4m3_encode(x)
    assert list(C.e4m3_decode(enc)) == [448, 448, 448, 448, -448, -448]
    assert np.all((enc & 0x7F) != 0x7F)


def test_bf16_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32),
                        (rng.standard_normal(50000) * 1e-30).astype(np.float32),
                        rng.integers(0, 2 ** 31, 50000, dtype=np.uint32).view(np.float32)])
    x = x[np.isfinite(x) & (np.abs(x) < 3e38)]
    ours = C.bf16_encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(C.bf16_decode(ours),
                          torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())


def test_e2m1_table_and_ties():
    with open(os.path.join(GOLDEN, "ocp_mx_e2m1.json")) as f:
        g = json.load(f)
    for item in g["codes"]:
        assert C.e2m1_decode(np.uint8(item["code"])) == item["value"]
    for item in g["ties"]:
        assert C.e2m1_decode(C.e2m1_encode(item["x"])) == item["value"], item


def test_e2m1_nearest_bruteforce():
    rng = np.random.default_rng(3)
    vals = C.e2m1_decode(np.arange(16))
    x = np.concatenate([rng.uniform(-7, 7, 4000), np.arange(-6.5, 6.5, 0.125)])
    enc = C.e2m1_encode(x)
    for xi, ci in zip(x, enc):
        xs = min(max(xi, -6.0), 6.0)
        d = np.abs(vals - xs)
        cands = [c for c in range(16) if d[c] == d.min()]
        if len(cands) > 1:
            cands = [c for c in cands if c & 1 == 0] or cands
        assert C.e2m1_decode(ci) in [C.e2m1_decode(c) for c in cands]


def test_e8m0_scale_decode_matches_torch():
    b = np.arange(0, 255, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    packed = np.zeros((255, 16), dtype=np.uint8) | np.uint8(0x2)  # all elements = +1.0
    dec = C.mxfp4_decode(packed, b[:, None])
    assert np.array_equal(dec[:, 0], ref)


def test_mxfp4_group_rules():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((500, 128)) * 2.0 ** rng.integers(-20, 20, (500, 1))).astype(np.float32)
    x[3, 32:64] = 0.0                       # an all-zero group
    x[7, :32] = 0.0
    x[7, 5] = 6.0 * 2.0 ** 3 * 1.3          # amax not a power of two
    packed, sc = C.mxfp4_encode(x)
    assert packed.shape == (500, 64) and sc.shape == (500, 4)
    dec = C.mxfp4_decode(packed, sc)
    xs = x.astype(np.float64).reshape(500, 4, 32)
    amax = np.abs(xs).max(-1)
    e = sc.astype(np.int64) - 127
    for i in range(500):
        for j in range(4):
            a = amax[i, j]
            if a == 0:
                assert sc[i, j] == 0 and np.all(dec[i, 32 * j:32 * j + 32] == 0)
                continue
            # brute force: the shared exponent puts amax / 2**e into [4, 8)
            good = [t for t in range(-140, 140) if 4.0 <= a / 2.0 ** t < 8.0]
            assert e[i, j] == good[0]
            # every element is a nearest e2m1 point of x / 2**e (saturating at 6)
            grid = np.unique(np.abs(C.e2m1_decode(np.arange(16)))) * 2.0 ** e[i, j]
            for xv, dv in zip(xs[i, j], dec[i, 32 * j:32 * j + 32]):
                xc = min(abs(xv), 6.0 * 2.0 ** e[i, j])
                assert abs(abs(dv) - xc) == np.min(np.abs(grid - xc))
                assert dv == 0 or np.sign(dv) == np.sign(xv)


def test_mxfp4_packing_low_nibble_first():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1.0     # element 0 -> low nibble of byte 0
    x[0, 1] = -6.0    # element 1 -> high nibble of byte 0
    x[0, 31] = 4.0
    packed, sc = C.mxfp4_encode(x)
    # amax 6 -> e = floor(log2 6) - 2 = 0 -> scale byte 127
    assert sc[0, 0] == 127
    assert packed[0, 0] == (0x2 | (0xF << 4))
    assert packed[0, 15] == (0x6 << 4)


def test_fp8_entry_scale_and_error_bound():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((300, 512)) / np.sqrt(512)).astype(np.float32)
    y[0, :448] = 0.0
    codes, rope, s = C.fp8_entry_encode(y, 448)
    assert s[0] == 1.0 and np.all(codes[0] & 0x7F == 0)
    dec = C.e4m3_decode(codes) * s[:, None].astype(np.float64)
    x = y[:, :448].astype(np.float64)
    amax = np.abs(x).max(1)
    # scale is fp32(amax/448); the amax element decodes to +-amax within fp32 ulps
    assert np.array_equal(s[1:], (amax[1:] / 448.0).astype(np.float32))
    col = np.argmax(np.abs(x[1:]), 1)
    assert np.allclose(np.abs(dec[np.arange(1, 300), col]), amax[1:], rtol=1e-6)
    # e4m3 half-spacing bound: relative 2**-4 in normals, absolute 2**-10 * s below
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s[:, None])
    assert np.all(np.abs(dec - x) <= bound * (1 + 1e-6))
    assert np.array_equal(rope, torch.from_numpy(y[:, 448:]).to(torch.bfloat16)
                          .view(torch.int16).numpy().view(np.uint16))


def test_kv_decode_rows_fp8_against_library_decode():
    # the FP8 branch of the cache-row decoder against an independent decode:
    # torch's float8_e4m3fn cast of the stored codes times the stored fp32
    # scale, and the RoPE dims through torch's bfloat16; the decoded rows lie
    # within the e4m3 half-spacing of the encoded values (a dropped, inverted
    # or misplaced scale fails both)
    rng = np.random.default_rng(17)
    y = (rng.standard_normal((2, 40, 512)) / np.sqrt(512)).astype(np.float32)
    y[1, 3] *= 1e3
    y[0, 5, :448] = 0.0
    kv = C.kv_encode(y, "fp8", 448)
    rows = np.array([0, 3, 5, 39, 7, 3])
    for b in range(2):
        got = C.kv_decode_rows(kv, b, rows)
        codes = torch.from_numpy(kv.nope[b, rows].copy()).view(torch.float8_e4m3fn)
        lib_nope = codes.to(torch.float64).numpy() * kv.scale[b, rows].astype(np.float64)[:, None]
        lib_rope = (torch.from_numpy(kv.rope[b, rows].copy().view(np.int16)).view(torch.bfloat16)
                    .to(torch.float64).numpy())
        assert np.array_equal(got[:, :448], lib_nope)
        assert np.array_equal(got[:, 448:], lib_rope)
        x = y[b, rows].astype(np.float64)
        s = kv.scale[b, rows].astype(np.float64)[:, None]
        bound = np.maximum(np.abs(x[:, :448]) * 2.0 ** -4, 2.0 ** -10 * s)
        assert np.all(np.abs(got[:, :448] - x[:, :448]) <= bound * (1 + 1e-6))
        assert np.all(np.abs(got[:, 448:] - x[:, 448:]) <= np.abs(x[:, 448:]) * 2.0 ** -8)
    assert np.all(C.kv_decode_rows(kv, 0, [5])[0, :448] == 0.0)
