"""Test-side helpers: move oracle arrays to and from the GPU, and the parity
rules the GPU path is held to.

Rules
  * outputs (attend): for every row (b, query, head),
        max |gpu - oracle| / max |oracle| <= 2e-2
    (bf16 output, fp32 accumulation); oracle = float64.
  * top-k: bit-exact index sets, except where the oracle's k'-th and
    (k'+1)-th scores (desc score, asc id order) differ by less than 1e-5
    relative -- then every id clearly above the boundary must be present and
    the rest may come from the tie band.
  * quantised caches (compress): decoded values equal, except elements whose
    pre-rounding value lies within QTOL (relative) of a rounding boundary
    (either neighbour accepted), and MXFP4 groups whose amax lies within QTOL
    of a scale-exponent boundary.  QTOL = 3e-5 covers the fp32 (GPU) versus
    float64 (oracle) evaluation of a softmax over up to 2m = 256 slots.
"""

import numpy as np
import torch

from long_context_attention_v4attn_amd import binding as B
from oracle import codecs as C
from oracle.indexer import topk_from_scores

OUT_TOL = 2e-2
TOPK_REL = 1e-5
QTOL = 3e-5


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def kv_to_dev(kv):
    if kv.fmt == "f32":
        return B.KVCache(B.F32, kv.d_nope, kv.d_rope, dev(kv.nope), dev(kv.rope))
    return B.KVCache(B.KV_FP8_BF16ROPE, kv.d_nope, kv.d_rope, dev(kv.nope),
                     dev(kv.rope.view(np.int16)).view(torch.bfloat16), dev(kv.scale))


def idx_to_dev(ix):
    if ix.fmt == "f32":
        return B.IdxCache(B.F32, ix.d, dev(ix.codes))
    return B.IdxCache(B.IDX_MXFP4, ix.d, dev(ix.codes), dev(ix.scales))


def kv_from_dev(kvd):
    if kvd.fmt == B.F32:
        return C.KV("f32", kvd.d_nope, kvd.d_rope, kvd.nope.cpu().numpy(), kvd.rope.cpu().numpy())
    return C.KV("fp8", kvd.d_nope, kvd.d_rope, kvd.nope.cpu().numpy(),
                kvd.rope.view(torch.int16).cpu().numpy().view(np.uint16), kvd.scale.cpu().numpy())


def idx_from_dev(ixd):
    if ixd.fmt == B.F32:
        return C.Idx("f32", ixd.d, ixd.codes.cpu().numpy())
    return C.Idx("mxfp4", ixd.d, ixd.codes.cpu().numpy(), ixd.scales.cpu().numpy())


def bf16_dev(x32):
    """float32 numpy -> bf16 device tensor with the oracle's rounding."""
    return dev(C.bf16_encode(x32).view(np.int16)).view(torch.bfloat16)


# ---------------------------------------------------------------- outputs

def out_to_f64(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def check_out(gpu, ref, tol=OUT_TOL, what="out"):
    """gpu, ref: [..., D]; per-row max abs error over max abs reference."""
    g = out_to_f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r).max(axis=-1)
    scale = np.abs(r).max(axis=-1)
    zero = scale == 0
    assert np.all(err[zero] == 0), f"{what}: nonzero output where the reference is 0"
    rel = np.where(zero, 0.0, err / np.where(zero, 1.0, scale))
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= tol, f"{what}: max row rel err {worst:.3e} > {tol}"
    return worst


# ---------------------------------------------------------------- top-k

def check_topk_row(gpu_row, scores, k):
    """gpu_row: int array [k]; scores: oracle float64 scores over n_vis blocks."""
    n = len(scores)
    kk = min(k, n)
    g = np.asarray(gpu_row, np.int64)
    assert np.all(g[kk:] == -1), "padding must be -1"
    sel = g[:kk]
    assert np.all(np.diff(sel) > 0), "ids must be ascending and unique"
    assert kk == 0 or (sel[0] >= 0 and sel[-1] < n), "ids out of range"
    s32 = C.f32(scores).astype(np.float64)
    order = sorted(range(n), key=lambda i: (-s32[i], i))
    ref = np.array(sorted(order[:kk]), np.int64)
    if kk == n or np.array_equal(sel, ref):
        return "exact"
    tk = s32[order[kk - 1]]
    tk1 = s32[order[kk]]
    eps = TOPK_REL * abs(tk)
    assert tk - tk1 < eps or tk == tk1, \
        f"top-k differs with a clear gap: tau_k={tk!r} tau_k+1={tk1!r}"
    sc = np.asarray(scores, np.float64)
    upper = set(np.nonzero(sc > tk + eps)[0].tolist())
    band = set(np.nonzero(np.abs(sc - tk) <= eps)[0].tolist())
    gs = set(sel.tolist())
    assert upper <= gs, "an id clearly above the boundary is missing"
    assert gs <= upper | band, "an id clearly below the boundary was selected"
    return "band"


def check_topk_row_bf16(gpu_row, scores, k):
    """The BF16-score selector.  Exact against the oracle's bf16 ranking,
    unless an id's fp32 score lies within TOPK_REL (relative) of a bf16
    rounding boundary -- the GPU's fp32 sum (another accumulation order) may
    round it to the neighbouring bf16 value; then ids certainly above the
    k-th bf16 value must be selected, ids certainly below must not, and ids
    at (or possibly at) that value may go either way."""
    n = len(scores)
    kk = min(k, n)
    g = np.asarray(gpu_row, np.int64)
    assert np.all(g[kk:] == -1), "padding must be -1"
    sel = g[:kk]
    assert np.all(np.diff(sel) > 0), "ids must be ascending and unique"
    assert kk == 0 or (sel[0] >= 0 and sel[-1] < n), "ids out of range"
    ref = topk_from_scores(scores, k, "bf16")[:kk]
    if kk == n or np.array_equal(sel, ref):
        return "exact"
    s32 = C.f32(scores).astype(np.float64)
    b = C.bf16_decode(C.bf16_encode(s32))
    lo = C.bf16_decode(C.bf16_encode(C.f32(s32 * (1 - TOPK_REL)))).astype(np.float64)
    hi = C.bf16_decode(C.bf16_encode(C.f32(s32 * (1 + TOPK_REL)))).astype(np.float64)
    vmin, vmax = np.minimum(np.minimum(lo, hi), b), np.maximum(np.maximum(lo, hi), b)
    amb = (vmin != b) | (vmax != b)
    order = sorted(range(n), key=lambda i: (-b[i], i))
    T = b[order[kk - 1]]
    assert np.any(amb & (vmax >= T) & (vmin <= T)), \
        "bf16 top-k differs with no score near a bf16 rounding boundary at the k-th value"
    gs = set(sel.tolist())
    above = set(np.nonzero(vmin > T)[0].tolist())
    below = set(np.nonzero(vmax < T)[0].tolist())
    assert above <= gs, "an id certainly above the k-th bf16 value is missing"
    assert not (gs & below), "an id certainly below the k-th bf16 value was selected"
    return "band"


# ---------------------------------------------------------------- quantised caches

def _ambiguous_e4m3(u):
    lo = C.e4m3_decode(C.e4m3_encode(np.clip(u * (1 - QTOL), -448, 448)))
    hi = C.e4m3_decode(C.e4m3_encode(np.clip(u * (1 + QTOL), -448, 448)))
    return lo != hi


def check_fp8_rows(gpu_kv, y, d_nope, rows=None):
    """gpu_kv: oracle-layout KV read back; y: oracle pooled rows float64 [B][n][D]."""
    codes, rope, s = C.fp8_entry_encode(y, d_nope)
    gs = gpu_kv.scale.astype(np.float64)
    rs = s.astype(np.float64)
    assert np.all(np.abs(gs - rs) <= QTOL * rs), "FP8 entry scales differ"
    gdec = C.e4m3_decode(gpu_kv.nope)
    rdec = C.e4m3_decode(codes)
    diff = gdec != rdec
    if np.any(diff):
        u = C.f32(y[..., :d_nope]).astype(np.float64) / rs[..., None]
        amb = _ambiguous_e4m3(u)
        assert np.all(amb[diff]), f"{int((diff & ~amb).sum())} FP8 codes differ away from a rounding boundary"
    gr = C.bf16_decode(gpu_kv.rope)
    rr = C.bf16_decode(rope)
    rdiff = gr != rr
    if np.any(rdiff):
        # bf16 RoPE dims: neighbours only where fp32 rounding decides
        assert np.all(np.abs(gr - rr)[rdiff] <= np.abs(rr[rdiff]) * 2.0 ** -7), "bf16 dims differ"


def check_mxfp4_rows(gpu_ix, y):
    """gpu_ix: oracle-layout Idx read back; y: float64 [B][n][d]."""
    codes, scales = C.mxfp4_encode(y)
    Bn, n, d = y.shape
    g = y.reshape(Bn, n, d // 32, 32)
    amax = np.abs(g).max(-1)
    _, k1 = np.frexp(amax * (1 - QTOL))
    _, k2 = np.frexp(amax * (1 + QTOL))
    edge = k1 != k2
    sc_ok = (gpu_ix.scales == scales) | edge
    assert np.all(sc_ok), "MXFP4 scales differ away from an exponent boundary"
    gdec = C.mxfp4_decode(gpu_ix.codes, gpu_ix.scales).reshape(Bn, n, d // 32, 32)
    rdec = C.mxfp4_decode(codes, scales).reshape(Bn, n, d // 32, 32)
    diff = (gdec != rdec) & ~edge[..., None]
    if np.any(diff):
        e = scales.astype(np.int64) - 127
        u = g * np.ldexp(1.0, -e)[..., None]
        lo = C.e2m1_decode(C.e2m1_encode(u * (1 - QTOL)))
        hi = C.e2m1_decode(C.e2m1_encode(u * (1 + QTOL)))
        amb = lo != hi
        assert np.all(amb[diff]), f"{int((diff & ~amb).sum())} FP4 codes differ away from a rounding boundary"


def check_f32_rows(gpu, y, rtol=QTOL):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(y, np.float64)
    scale = np.abs(r).max(axis=-1, keepdims=True) + 1e-30
    assert np.all(np.abs(g - r) <= rtol * scale), "fp32 rows differ"
