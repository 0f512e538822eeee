"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every function include/v4attn.h declares; helpers answer; invalid arguments are
rejected on the host before anything is enqueued."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "v4attn.h")


@pytest.fixture(scope="module")
def clib():
    from long_context_attention_v4attn_amd import binding
    if not os.path.exists(binding.library_path()):
        from long_context_attention_v4attn_amd import build
        build.build()
    return binding.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(v4attn_\w+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("v4attn_compress", "v4attn_index_topk", "v4attn_csa_attend", "v4attn_hca_attend"):
        assert n in names


def test_library_exports_every_declared_symbol(clib):
    for name in _declared():
        assert hasattr(clib, name), f"{name} not exported"


def test_status_strings_and_version(clib):
    from long_context_attention_v4attn_amd import binding as B
    for s in (0, -1, -2, -3, -4, -5):
        assert B.v4attn_status_str(s)
    assert clib.v4attn_version() >= 100
    assert clib.v4attn_last_hip_error() == 0


def test_workspace_sizes(clib):
    from long_context_attention_v4attn_amd import binding as B
    # scores [R][cap] fp32 plus the quantised queries
    n = B.v4attn_workspace_bytes(B.OP_INDEX_TOPK, 4, 1, 16, 128, 262144, 2048, 0)
    assert n >= 4 * 262144 * 4
    # a short entry list needs no split partials
    assert B.v4attn_workspace_bytes(B.OP_CSA_ATTEND, 1, 1, 64, 512, 0, 32, 32) == 0
    # a long one does, and the need does not depend on B per query
    a = B.v4attn_workspace_bytes(B.OP_HCA_ATTEND, 1, 1, 64, 512, 8192, 128, 128)
    b = B.v4attn_workspace_bytes(B.OP_HCA_ATTEND, 16, 1, 64, 512, 8192, 128, 128)
    assert a > 0 and b >= 16 * a - 16 * 512
    # the fused call's index workspace adds the selector's per-chunk lists
    # (8 bytes per key row and query)
    f = B.v4attn_workspace_bytes(B.OP_CSA_INDEX, 4, 1, 16, 128, 262144, 2048, 0)
    assert f >= n + 4 * 262144 * 8
    with pytest.raises(B.V4AttnError):
        B.v4attn_workspace_bytes(99, 1, 1, 1, 1, 1, 1, 1)


class _KV(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("_pad", ctypes.c_int32), ("cap", ctypes.c_int64), ("nope", ctypes.c_void_p),
                ("rope", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class _Idx(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("d", ctypes.c_int32), ("cap", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def test_invalid_arguments_rejected_on_host(clib):
    kv = _KV(2, 448, 64, 0, 100, 0x1000, 0x2000, 0x3000)
    r = ctypes.byref
    # compress: null input, bad m, T not a multiple of m, mismatched dims
    assert clib.v4attn_compress(None, None, None, None, None, 0, 1, 4, 512, 4, 0, 0, r(kv), None) == -1
    assert clib.v4attn_compress(FAKE, None, None, None, None, 0, 1, 6, 512, 3, 0, 0, r(kv), None) == -2
    assert clib.v4attn_compress(FAKE, None, None, None, None, 0, 1, 6, 512, 4, 0, 0, r(kv), None) == -1
    assert clib.v4attn_compress(FAKE, None, None, None, None, 0, 1, 8, 500, 4, 0, 0, r(kv), None) == -1
    assert clib.v4attn_compress(FAKE, None, None, FAKE, None, 0, 1, 8, 512, 4, 0, 0, r(kv), None) == -1
    # index_topk: k = 0, unsupported d, missing workspace
    ix = _Idx(3, 128, 1000, 0x1000, 0x2000)
    assert clib.v4attn_index_topk(FAKE, 1, FAKE, r(ix), FAKE, 1, 1, 16, 4, 0, FAKE, FAKE, 1 << 30, None) == -1
    ix_bad = _Idx(3, 64, 1000, 0x1000, 0x2000)
    assert clib.v4attn_index_topk(FAKE, 1, FAKE, r(ix_bad), FAKE, 1, 1, 16, 4, 8, FAKE, FAKE, 1 << 30, None) == -2
    assert clib.v4attn_index_topk(FAKE, 1, FAKE, r(ix), FAKE, 1, 1, 16, 4, 8, FAKE, None, 0, None) == -3
    # the BF16-score variant validates the same way
    assert clib.v4attn_index_topk_bf16(FAKE, 1, FAKE, r(ix), FAKE, 1, 1, 16, 4, 0, FAKE, FAKE, 1 << 30, None) == -1
    assert clib.v4attn_index_topk_bf16(FAKE, 1, FAKE, r(ix_bad), FAKE, 1, 1, 16, 4, 8, FAKE, FAKE, 1 << 30,
                                       None) == -2
    assert clib.v4attn_index_topk_bf16(FAKE, 1, FAKE, r(ix), FAKE, 1, 1, 16, 4, 8, FAKE, None, 0, None) == -3
    # the allocation-free variant: the same validation, and a call that needs
    # more than its fixed scratch (28 rows over 262144 blocks) -> -5, all on
    # the host (nothing is read or enqueued)
    assert clib.v4attn_index_topk_noalloc(FAKE, 1, FAKE, r(ix), FAKE, 1, 1, 16, 4, 0, FAKE, None) == -1
    assert clib.v4attn_index_topk_noalloc(FAKE, 1, FAKE, r(ix_bad), FAKE, 1, 1, 16, 4, 8, FAKE, None) == -2
    ix_1m = _Idx(3, 128, 262144, 0x1000, 0x2000)
    assert clib.v4attn_index_topk_noalloc(FAKE, 1, FAKE, r(ix_1m), FAKE, 28, 1, 16, 4, 2048, FAKE, None) == -5
    # attend: H not a multiple of 16 on the FP8 path, window ring too small, f32 q on FP8
    win = _KV(2, 448, 64, 0, 64, 0x1000, 0x2000, 0x3000)
    assert clib.v4attn_hca_attend(FAKE, 1, r(kv), 128, r(kv), 16, FAKE, None, ctypes.c_float(0.1),
                                  1, 1, 24, FAKE, 1, FAKE, 1 << 30, None) == -2
    assert clib.v4attn_hca_attend(FAKE, 1, r(kv), 128, r(win), 128, FAKE, None, ctypes.c_float(0.1),
                                  1, 1, 64, FAKE, 1, FAKE, 1 << 30, None) == -1
    assert clib.v4attn_csa_attend(FAKE, 0, r(kv), FAKE, 8, r(kv), 16, FAKE, None, ctypes.c_float(0.1),
                                  1, 1, 64, FAKE, 1, FAKE, 1 << 30, None) == -2
    # format mismatch between cache and ring
    kv32 = _KV(0, 448, 64, 0, 100, 0x1000, 0x2000, 0)
    assert clib.v4attn_csa_attend(FAKE, 1, r(kv), FAKE, 8, r(kv32), 16, FAKE, None, ctypes.c_float(0.1),
                                  1, 1, 64, FAKE, 1, FAKE, 1 << 30, None) == -1
    # a long entry list needs split partials: no workspace -> -3
    big = _KV(2, 448, 64, 0, 10000, 0x1000, 0x2000, 0x3000)
    assert clib.v4attn_hca_attend(FAKE, 1, r(big), 4, r(kv), 16, FAKE, None, ctypes.c_float(0.1),
                                  1, 1, 64, FAKE, 1, None, 0, None) == -3
    # the fused index + CSA call: the index call's checks (k = 0), the
    # attend call's (f32 q on FP8 entries), a missing index workspace
    fused = clib.v4attn_csa_index_attend
    assert fused(FAKE, 1, FAKE, r(ix), 16, 4, 0, FAKE, FAKE, 1, r(kv), r(kv), 16, FAKE, None,
                 ctypes.c_float(0.1), 1, 1, 64, FAKE, 1, FAKE, 1 << 30, FAKE, 1 << 30, None) == -1
    assert fused(FAKE, 1, FAKE, r(ix), 16, 4, 8, FAKE, FAKE, 0, r(kv), r(kv), 16, FAKE, None,
                 ctypes.c_float(0.1), 1, 1, 64, FAKE, 1, FAKE, 1 << 30, FAKE, 1 << 30, None) == -2
    assert fused(FAKE, 1, FAKE, r(ix), 16, 4, 8, FAKE, FAKE, 1, r(kv), r(kv), 16, FAKE, None,
                 ctypes.c_float(0.1), 1, 1, 64, FAKE, 1, None, 0, FAKE, 1 << 30, None) == -3


class _NR(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("inv_freq", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("_pad", ctypes.c_int32)]


def test_norm_rope_variants_rejected_on_host(clib):
    from long_context_attention_v4attn_amd import binding as B
    r = ctypes.byref
    nr = _NR(0x4000, 0x5000, 1e-6, 0)
    bad = _NR(0x4000, 0x5000, -1.0, 0)
    kv = _KV(2, 448, 64, 0, 100, 0x1000, 0x2000, 0x3000)
    kv32 = _KV(0, 448, 64, 0, 100, 0x1000, 0x2000, 0)
    ix = _Idx(3, 128, 1000, 0x1000, 0x2000)
    # compress: indexer keys take no norm/RoPE; negative eps
    assert clib.v4attn_compress_nr(FAKE, None, None, None, None, 0, 1, 4, 128, 4, 0, 1, r(ix), r(nr),
                                   None) == -2
    assert clib.v4attn_compress_nr(FAKE, None, None, None, None, 0, 1, 4, 512, 4, 0, 0, r(kv), r(bad),
                                   None) == -1
    # attend: FP8 entries only; negative eps; the plain-call checks still apply
    assert clib.v4attn_csa_attend_nr(FAKE, 1, r(kv32), FAKE, 8, r(kv32), 16, FAKE, None,
                                     ctypes.c_float(0.1), 1, 1, 64, FAKE, 1, r(nr), FAKE, 1 << 30,
                                     None) == -2
    assert clib.v4attn_hca_attend_nr(FAKE, 1, r(kv), 128, r(kv), 16, FAKE, None, ctypes.c_float(0.1),
                                     1, 1, 64, FAKE, 1, r(bad), FAKE, 1 << 30, None) == -1
    assert clib.v4attn_hca_attend_nr(FAKE, 1, r(kv), 128, r(kv), 16, FAKE, None, ctypes.c_float(0.1),
                                     1, 1, 24, FAKE, 1, r(nr), FAKE, 1 << 30, None) == -2
    # the _nr calls normalise the queries inside the attention kernel: the
    # same workspace as the plain calls
    for op, op_nr in ((B.OP_CSA_ATTEND, B.OP_CSA_ATTEND_NR), (B.OP_HCA_ATTEND, B.OP_HCA_ATTEND_NR)):
        a = B.v4attn_workspace_bytes(op, 4, 1, 64, 512, 8192, 2048, 128)
        b = B.v4attn_workspace_bytes(op_nr, 4, 1, 64, 512, 8192, 2048, 128)
        assert b == a


class _Pg(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("page_tokens", ctypes.c_int32)]


def test_paged_variants_rejected_on_host(clib):
    r = ctypes.byref
    f = ctypes.c_float(0.1)
    pg = _Pg(0x6000, 8, 512)                     # 128 CSA entries per page
    kv = _KV(2, 448, 64, 0, 128 * 10, 0x1000, 0x2000, 0x3000)     # a pool of 10 pages
    kv32 = _KV(0, 448, 64, 0, 128 * 10, 0x1000, 0x2000, 0)
    ix = _Idx(3, 128, 128 * 10, 0x1000, 0x2000)
    ix32 = _Idx(0, 128, 128 * 10, 0x1000, 0)

    def csa(comp, pages, m=4):
        return clib.v4attn_csa_attend_paged(FAKE, 1, r(comp), r(pages) if pages else None, m, FAKE,
                                            8, r(comp), 16, FAKE, None, f, 1, 1, 64, FAKE, 1, None,
                                            FAKE, 1 << 30, None)

    def idx(keys, pages, m=4):
        return clib.v4attn_index_topk_paged(FAKE, 1, FAKE, r(keys), r(pages) if pages else None,
                                            FAKE, 1, 1, 16, m, 64, 0, FAKE, FAKE, 1 << 30, None)
    # no table; page sizes that are not powers of two >= 128
    assert csa(kv, None) == -1
    for bad in (_Pg(0x6000, 8, 192), _Pg(0x6000, 8, 64), _Pg(0x6000, 0, 512), _Pg(None, 8, 512)):
        assert csa(kv, bad) in (-1, -2)
    # fp32 caches are not paged; m above the page
    assert csa(kv32, pg) == -2
    assert csa(kv, pg, m=1024) == -2
    # the pool is not whole pages
    assert csa(_KV(2, 448, 64, 0, 1000, 0x1000, 0x2000, 0x3000), pg) == -1
    # indexer: MXFP4 keys with >= 128 keys per page only
    assert idx(ix, _Pg(0x6000, 8, 256)) == -2
    assert idx(ix32, pg) == -2
    assert idx(ix, None) == -1
    # HCA: rate 128 on 512-token pages is 4 entries per page (accepted shape);
    # a pool that is not whole pages is still refused
    assert clib.v4attn_hca_attend_paged(FAKE, 1, r(_KV(2, 448, 64, 0, 6, 0x1000, 0x2000, 0x3000)),
                                        r(pg), 128, r(kv), 16, FAKE, None, f, 1, 1, 64, FAKE, 1,
                                        None, FAKE, 1 << 30, None) == -1
    # compress: the call's blocks past the sequence's pages
    assert clib.v4attn_compress_paged(FAKE, None, None, None, None, 0, 1, 4 * 1100, 512, 4, 0, 0,
                                      r(kv), r(pg), None, None) == -1
    # append: a rate above 1 (or overlap) needs the pooling state
    def app(state, m=4, kv_prev=None):
        return clib.v4attn_append(FAKE, None, kv_prev, None, state, FAKE, None, 0, 2, 512, m, 0,
                                  r(kv), r(pg), None, None)
    assert app(None) == -1
    assert app(None, m=1, kv_prev=FAKE) == -1
    assert app(FAKE, m=256) == -2                                   # above the page size
    assert clib.v4attn_append(FAKE, None, None, None, None, None, None, 0, 2, 512, 1, 0, r(kv),
                              None, None, None) == -1                 # no positions


def test_append_batch_rejected_on_host(clib):
    from long_context_attention_v4attn_amd.binding import _Append
    r = ctypes.byref
    kv = _KV(2, 448, 64, 0, 100, 0x1000, 0x2000, 0x3000)
    assert clib.v4attn_append_batch(0, None, None) == 0
    assert clib.v4attn_append_batch(1, None, None) == -1
    assert clib.v4attn_append_batch(-1, None, None) == -1
    arr = (_Append * 9)()
    assert clib.v4attn_append_batch(9, arr, None) == -2          # more than V4A_MAX_APPEND
    # one bad call (rate 4 without a state) refuses the whole batch
    good = _Append(0x1000, None, None, None, None, 0x5000, None, ctypes.cast(ctypes.pointer(kv), ctypes.c_void_p),
                   None, None, 0, 2, 512, 1, 0, 0)
    bad = _Append(0x1000, None, None, None, None, 0x5000, None, ctypes.cast(ctypes.pointer(kv), ctypes.c_void_p),
                  None, None, 0, 2, 512, 4, 0, 0)
    two = (_Append * 2)(good, bad)
    assert clib.v4attn_append_batch(2, two, None) == -1


def test_empty_calls_need_no_pointers(clib):
    # B == 0 (or Q == 0, or T == 0 for the chunked compressor): V4A_OK without
    # reading any data pointer (torch hands out NULL for empty tensors)
    f = ctypes.c_float(0.1)
    assert clib.v4attn_compress(None, None, None, None, None, 0, 0, 4, 512, 4, 0, 0, None, None) == 0
    assert clib.v4attn_compress(None, None, None, None, None, 0, 2, 0, 512, 4, 0, 0, None, None) == 0
    assert clib.v4attn_append(None, None, None, None, None, None, None, 0, 0, 512, 4, 0, None, None,
                              None, None) == 0
    assert clib.v4attn_index_topk(None, 1, None, None, None, 0, 1, 16, 4, 64, None, None, 0,
                                  None) == 0
    assert clib.v4attn_index_topk_paged(None, 1, None, None, None, None, 2, 0, 16, 4, 64, 0, None,
                                        None, 0, None) == 0
    assert clib.v4attn_csa_attend(None, 1, None, None, 8, None, 16, None, None, f, 0, 1, 64, None, 1,
                                  None, 0, None) == 0
    assert clib.v4attn_hca_attend_paged(None, 1, None, None, 128, None, 16, None, None, f, 3, 0, 64,
                                        None, 1, None, None, 0, None) == 0
    # negative sizes stay invalid
    assert clib.v4attn_index_topk(None, 1, None, None, None, -1, 1, 16, 4, 64, None, None, 0,
                                  None) == -1


def test_binding_refuses_host_tensors():
    import numpy as np
    import torch
    from long_context_attention_v4attn_amd import binding as B
    try:
        B.load()
    except B.V4AttnError:
        pytest.skip("library not built")
    x = torch.zeros(1, 4, 512)
    out = B.KVCache(B.F32, 448, 64, torch.zeros(1, 2, 448), torch.zeros(1, 2, 64))
    with pytest.raises(B.V4AttnError):
        B.v4attn_compress(x, None, None, None, None, 4, 0, out)
