"""Number formats of the cache and the indexer (oracle; test infrastructure).

Storage precisions come from [Notes §9] ("KV storage precision": RoPE
dimensions in BF16, every other KV dimension in FP8) and [Notes §9] / [HF
"Hybrid attention"] (the lightning indexer runs in FP4).  The pages do not fix
the scale granularity; the readings used here are

* FP8 attention entry: one fp32 scale per entry, s = fp32(amax / 448) over the
  d_nope non-RoPE dimensions (s = 1 when amax = 0), code = e4m3fn(x / s) with
  saturation at +-448 -- the "per-token scale" of the benchmark configurations.
* FP4 indexer vectors: OCP MXFP4, groups of 32 consecutive elements sharing an
  e8m0 scale 2**e with e = floor(log2 amax) - 2 ([OCP-MX] shared-exponent
  rule, emax(e2m1) = 2), elements e2m1 with round-to-nearest-even and
  saturation at +-6.

Both scale rules are conventions: "parity unpinned" by the pages (no page
prints a scale or a quantised value); they are pinned here only against the
OCP definitions and library casts (torch float8_e4m3fn / bfloat16).

Layouts (shared with the C ABI, row-major):
  KV  (fmt "f32"):  nope f32 [B][cap][d_nope], rope f32 [B][cap][d_rope]
  KV  (fmt "fp8"):  nope u8 e4m3fn [B][cap][d_nope], rope u16 bf16 bits
                    [B][cap][d_rope], scale f32 [B][cap]
  Idx (fmt "f32"):  codes f32 [B][cap][d]
  Idx (fmt "mxfp4"): codes u8 [B][cap][d/2] (element 2i in the low nibble),
                    scales u8 e8m0 [B][cap][d/32]
"""

from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------- fp32 / bf16


def f32(x):
    """Round float64 values to the nearest fp32 (IEEE RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_encode(x):
    """fp32 -> bf16 bits, round to nearest even on the 16 dropped bits."""
    v = np.asarray(x, dtype=np.float32)
    assert np.all(np.isfinite(v)), "bf16_encode: non-finite input"
    u = v.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_decode(bits):
    """bf16 bits -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- e4m3fn
# [OCP-FP8] E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
# S.1111.111 is NaN; largest finite 448; subnormal quantum 2**-9.

E4M3_MAX = 448.0


def e4m3_decode_table():
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sgn = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        mnt = c & 0x7
        if e == 0xF and mnt == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sgn * mnt * 2.0 ** -9
        else:
            t[c] = sgn * (1.0 + mnt / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3_TABLE = e4m3_decode_table()


def e4m3_decode(codes):
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def _rne_to_grid(a, mbits, emin):
    """Round magnitudes a >= 0 to a float grid with `mbits` mantissa bits
    whose smallest normal binade is 2**emin (subnormals share its quantum)."""
    _, k = np.frexp(a)                      # a = f * 2**k, f in [0.5, 1)
    e = np.maximum(k - 1, emin)             # binade exponent floor(log2 a)
    q = np.ldexp(1.0, e - mbits)            # spacing of the grid in that binade
    return np.rint(a / q) * q               # np.rint: round half to even


def e4m3_encode(x):
    """Values (already divided by the scale, in fp32) -> e4m3fn codes.
    Saturates to +-448, rounds to nearest even, never produces NaN."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x))
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    v = np.minimum(_rne_to_grid(a, 3, -6), E4M3_MAX)
    _, k = np.frexp(v)
    e = k - 1
    normal = v >= 2.0 ** -6
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, v / np.ldexp(1.0, np.where(normal, e, 0)) * 8.0 - 8.0,
                    v / 2.0 ** -9)
    code = (neg.astype(np.int64) << 7) | (exp_field.astype(np.int64) << 3) | \
        np.rint(mant).astype(np.int64)
    return code.astype(np.uint8)


# ---------------------------------------------------------------- e2m1
# [OCP-MX] FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
# {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no NaN / infinity.

E2M1_MAX = 6.0
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(nibbles):
    n = np.asarray(nibbles, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[n & 0x7]
    return np.where(n & 0x8, -mag, mag)


def e2m1_encode(x):
    """Values -> 4-bit codes (uint8 holding 0..15); RNE, saturating at +-6."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x))
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E2M1_MAX)
    v = np.minimum(_rne_to_grid(a, 1, 0), E2M1_MAX)
    # grid value -> magnitude code (index into E2M1_MAGNITUDES)
    idx = np.searchsorted(E2M1_MAGNITUDES, v)
    assert np.all(E2M1_MAGNITUDES[idx] == v)
    return ((neg.astype(np.uint8) << 3) | idx.astype(np.uint8)).astype(np.uint8)


# ---------------------------------------------------------------- MXFP4

MX_BLOCK = 32


def mxfp4_encode(x):
    """[..., d] values (fp32) -> (packed codes u8 [..., d/2], e8m0 u8 [..., d/32]).

    Per group of 32: amax = 0 gives scale byte 0 and zero codes; otherwise
    e = floor(log2 amax) - 2 clamped to [-127, 127], codes = e2m1(x * 2**-e).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    g = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(g), axis=-1)
    _, k = np.frexp(amax)
    e = np.clip(k - 1 - 2, -127, 127)
    e = np.where(amax > 0, e, -127)
    codes = e2m1_encode(g * np.ldexp(1.0, -e)[..., None])
    codes = np.where((amax > 0)[..., None], codes, 0).astype(np.uint8)
    codes = codes.reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def mxfp4_decode(packed, scales):
    """(packed u8 [..., d/2], e8m0 u8 [..., d/32]) -> float64 [..., d] (exact)."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = e2m1_decode(packed & 0xF)
    hi = e2m1_decode(packed >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    d = vals.shape[-1]
    sc = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    g = vals.reshape(vals.shape[:-1] + (d // MX_BLOCK, MX_BLOCK)) * sc[..., None]
    return g.reshape(vals.shape)


def mxfp4_roundtrip(x):
    return mxfp4_decode(*mxfp4_encode(x))


# ---------------------------------------------------------------- cache rows


@dataclass
class KV:
    """Attention entries: compressed cache or raw-token window ring."""
    fmt: str            # "f32" | "fp8"
    d_nope: int
    d_rope: int
    nope: np.ndarray    # f32 [B][cap][d_nope] | u8 [B][cap][d_nope]
    rope: np.ndarray    # f32 [B][cap][d_rope] | u16 bf16 bits [B][cap][d_rope]
    scale: np.ndarray = None   # None | f32 [B][cap]

    @property
    def cap(self):
        return self.nope.shape[1]

    @property
    def batch(self):
        return self.nope.shape[0]


@dataclass
class Idx:
    """Compressed lightning-indexer keys."""
    fmt: str            # "f32" | "mxfp4"
    d: int
    codes: np.ndarray   # f32 [B][cap][d] | u8 [B][cap][d/2]
    scales: np.ndarray = None  # None | u8 [B][cap][d/32]

    @property
    def cap(self):
        return self.codes.shape[1]


def fp8_entry_encode(y, d_nope):
    """fp32 rows [..., D] -> (e4m3 codes [..., d_nope], bf16 bits [..., D-d_nope], scale [...]).

    s = fp32(amax/448) (1 when amax = 0); code = e4m3fn(clamp(fp32(x/s), +-448));
    the RoPE tail is rounded to bf16 ([Notes §9], KV storage precision).
    """
    y = f32(y)
    nope = y[..., :d_nope].astype(np.float64)
    rope = y[..., d_nope:]
    amax = np.max(np.abs(nope), axis=-1)
    s = np.where(amax > 0, f32(amax / E4M3_MAX).astype(np.float64), 1.0)
    u = f32(nope / s[..., None]).astype(np.float64)
    u = np.clip(u, -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(u), bf16_encode(rope), f32(s)


def kv_encode(y, fmt, d_nope):
    """fp32 rows [B][n][D] -> KV with cap = n."""
    y = f32(y)
    if fmt == "f32":
        return KV("f32", d_nope, y.shape[-1] - d_nope, y[..., :d_nope].copy(),
                  y[..., d_nope:].copy(), None)
    codes, rope, s = fp8_entry_encode(y, d_nope)
    return KV("fp8", d_nope, y.shape[-1] - d_nope, codes, rope, s)


def kv_decode_rows(kv, b, rows):
    """Decoded entries (float64 [len(rows)][D]) of sequence b at cache rows."""
    rows = np.asarray(rows, dtype=np.int64)
    if kv.fmt == "f32":
        nope = kv.nope[b, rows].astype(np.float64)
        rope = kv.rope[b, rows].astype(np.float64)
    else:
        nope = e4m3_decode(kv.nope[b, rows]) * kv.scale[b, rows].astype(np.float64)[:, None]
        rope = bf16_decode(kv.rope[b, rows])
    return np.concatenate([nope, rope], axis=-1)


def idx_encode(y, fmt):
    y = f32(y)
    if fmt == "f32":
        return Idx("f32", y.shape[-1], y.copy(), None)
    codes, scales = mxfp4_encode(y)
    return Idx("mxfp4", y.shape[-1], codes, scales)


def idx_decode_rows(idx, b, rows):
    rows = np.asarray(rows, dtype=np.int64)
    if idx.fmt == "f32":
        return idx.codes[b, rows].astype(np.float64)
    return mxfp4_decode(idx.codes[b, rows], idx.scales[b, rows])
