"""ctypes binding of libv4attn.so (include/v4attn.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no fallback -- a missing library, a missing GPU or a failed call
raises V4AttnError.
"""

import ctypes
import os
from dataclasses import dataclass

import torch

F32, BF16, KV_FP8_BF16ROPE, IDX_MXFP4 = 0, 1, 2, 3
OUT_KV, OUT_IDX = 0, 1
OP_INDEX_TOPK, OP_CSA_ATTEND, OP_HCA_ATTEND = 1, 2, 3
OP_CSA_ATTEND_NR, OP_HCA_ATTEND_NR = 4, 5
OP_CSA_INDEX = 6

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class V4AttnError(RuntimeError):
    pass


def library_path():
    return os.environ.get("V4ATTN_LIB", os.path.join(_HERE, "libv4attn.so"))


class _KV(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("_pad", ctypes.c_int32),
                ("cap", ctypes.c_int64), ("nope", ctypes.c_void_p),
                ("rope", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class _NormRope(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("inv_freq", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("_pad", ctypes.c_int32)]


class _Pages(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("page_tokens", ctypes.c_int32)]


class _Append(ctypes.Structure):
    _fields_ = [("kv_cur", ctypes.c_void_p), ("gate_cur", ctypes.c_void_p),
                ("kv_prev", ctypes.c_void_p), ("gate_prev", ctypes.c_void_p),
                ("state", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("pos_bias", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("pages", ctypes.c_void_p), ("nr", ctypes.c_void_p),
                ("in_dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("d", ctypes.c_int32),
                ("m", ctypes.c_int32), ("out_kind", ctypes.c_int32), ("_pad", ctypes.c_int32)]


@dataclass
class NormRope:
    """[Notes §9] query / KV-entry RMSNorm and partial RoPE: gamma f32 [D]
    (None: no RMSNorm), inv_freq f32 [d_rope / 2] (None: no RoPE), eps."""
    gamma: object = None
    inv_freq: object = None
    eps: float = 1e-6

    def c_struct(self):
        _need_cuda(self.gamma, self.inv_freq)
        return _NormRope(_ptr(self.gamma), _ptr(self.inv_freq), float(self.eps), 0)


class _Idx(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("d", ctypes.c_int32),
                ("cap", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float

_SIGS = {
    "v4attn_compress": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I64, _I32, _P, _P]),
    "v4attn_index_topk": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "v4attn_index_topk_bf16": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ,
                                      _P]),
    "v4attn_index_topk_noalloc": (_I32, [_P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P]),
    "v4attn_csa_attend": (_I32, [_P, _I32, _P, _P, _I32, _P, _I32, _P, _P, _F, _I32, _I32, _I32,
                                 _P, _I32, _P, _SZ, _P]),
    "v4attn_csa_attend_nr": (_I32, [_P, _I32, _P, _P, _I32, _P, _I32, _P, _P, _F, _I32, _I32, _I32,
                                    _P, _I32, _P, _P, _SZ, _P]),
    "v4attn_hca_attend_nr": (_I32, [_P, _I32, _P, _I32, _P, _I32, _P, _P, _F, _I32, _I32, _I32,
                                    _P, _I32, _P, _P, _SZ, _P]),
    "v4attn_compress_nr": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I64, _I32, _P,
                                  _P, _P]),
    "v4attn_hca_attend": (_I32, [_P, _I32, _P, _I32, _P, _I32, _P, _P, _F, _I32, _I32, _I32,
                                 _P, _I32, _P, _SZ, _P]),
    "v4attn_compress_paged": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I64, _I32,
                                     _P, _P, _P, _P]),
    "v4attn_append": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P,
                             _P]),
    "v4attn_append_batch": (_I32, [_I32, _P, _P]),
    "v4attn_index_topk_paged": (_I32, [_P, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                       _P, _P, _SZ, _P]),
    "v4attn_csa_attend_paged": (_I32, [_P, _I32, _P, _P, _I32, _P, _I32, _P, _I32, _P, _P, _F, _I32,
                                       _I32, _I32, _P, _I32, _P, _P, _SZ, _P]),
    "v4attn_hca_attend_paged": (_I32, [_P, _I32, _P, _P, _I32, _P, _I32, _P, _P, _F, _I32, _I32,
                                       _I32, _P, _I32, _P, _P, _SZ, _P]),
    "v4attn_csa_index_attend": (_I32, [_P, _I32, _P, _P, _I32, _I32, _I32, _P, _P, _I32, _P, _P,
                                       _I32, _P, _P, _F, _I32, _I32, _I32, _P, _I32, _P, _SZ, _P,
                                       _SZ, _P]),
    "v4attn_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I64, _I32, _I32]),
    "v4attn_status_str": (ctypes.c_char_p, [_I32]),
    "v4attn_last_hip_error": (_I32, []),
    "v4attn_version": (_I32, []),
    "v4attn_time_next_kernel": (None, [_P, _P]),
}


def load():
    """Load libv4attn.so (idempotent); raises V4AttnError when it is absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise V4AttnError(f"libv4attn.so not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def v4attn_time_next_kernel(start, stop):
    """Record the raw hipEvent_t handles `start` / `stop` (ints) around the
    dominant kernel of this thread's next index / attend call."""
    load().v4attn_time_next_kernel(ctypes.c_void_p(start), ctypes.c_void_p(stop))


def v4attn_status_str(status):
    return load().v4attn_status_str(int(status)).decode()


def _check(status, what):
    if status != 0:
        lib = load()
        msg = lib.v4attn_status_str(status).decode()
        raise V4AttnError(f"{what}: {msg} (status {status}, hip error {lib.v4attn_last_hip_error()})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise V4AttnError(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise V4AttnError("tensors must be on the GPU (no host fallback)")


@dataclass
class KVCache:
    """Attention entries (compressed cache or window ring) in device memory."""
    fmt: int
    d_nope: int
    d_rope: int
    nope: torch.Tensor          # f32 [B][cap][d_nope] | uint8 e4m3fn [B][cap][d_nope]
    rope: torch.Tensor          # f32 [B][cap][d_rope] | bf16 [B][cap][d_rope]
    scale: torch.Tensor = None  # None | f32 [B][cap]

    @staticmethod
    def empty(B, cap, d_nope, d_rope, fmt, device="cuda"):
        if fmt == F32:
            return KVCache(F32, d_nope, d_rope,
                           torch.zeros(B, cap, d_nope, dtype=torch.float32, device=device),
                           torch.zeros(B, cap, d_rope, dtype=torch.float32, device=device))
        return KVCache(KV_FP8_BF16ROPE, d_nope, d_rope,
                       torch.zeros(B, cap, d_nope, dtype=torch.uint8, device=device),
                       torch.zeros(B, cap, d_rope, dtype=torch.bfloat16, device=device),
                       torch.ones(B, cap, dtype=torch.float32, device=device))

    @property
    def cap(self):
        return self.nope.shape[1]

    def c_struct(self):
        _need_cuda(self.nope, self.rope, self.scale)
        return _KV(self.fmt, self.d_nope, self.d_rope, 0, self.cap, self.nope.data_ptr(),
                   self.rope.data_ptr(), 0 if self.scale is None else self.scale.data_ptr())


@dataclass
class IdxCache:
    """Compressed lightning-indexer keys in device memory."""
    fmt: int
    d: int
    codes: torch.Tensor          # f32 [B][cap][d] | uint8 [B][cap][d/2]
    scales: torch.Tensor = None  # None | uint8 e8m0 [B][cap][d/32]

    @staticmethod
    def empty(B, cap, d, fmt, device="cuda"):
        if fmt == F32:
            return IdxCache(F32, d, torch.zeros(B, cap, d, dtype=torch.float32, device=device))
        return IdxCache(IDX_MXFP4, d, torch.zeros(B, cap, d // 2, dtype=torch.uint8, device=device),
                        torch.zeros(B, cap, d // 32, dtype=torch.uint8, device=device))

    @property
    def cap(self):
        return self.codes.shape[1]

    def c_struct(self):
        _need_cuda(self.codes, self.scales)
        return _Idx(self.fmt, self.d, self.cap, self.codes.data_ptr(),
                    0 if self.scales is None else self.scales.data_ptr())


def v4attn_workspace_bytes(op, B, Q, H, d, cap, k, n_win):
    n = load().v4attn_workspace_bytes(op, B, Q, H, d, cap, k, n_win)
    if n == ctypes.c_size_t(-1).value:
        raise V4AttnError("invalid workspace query")
    return n


def _workspace(ws, nbytes, device):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise V4AttnError("workspace too small")
    return ws, ws.numel() * ws.element_size()


def v4attn_compress(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, m, t0, out, stream=None):
    """Pool tokens [t0, t0+T) of every sequence into `out` (KVCache | IdxCache)."""
    lib = load()
    _need_cuda(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias)
    B, T, d = kv_cur.shape
    kind = OUT_KV if isinstance(out, KVCache) else OUT_IDX
    st = out.c_struct()
    s = lib.v4attn_compress(_ptr(kv_cur), _ptr(gate_cur), _ptr(kv_prev), _ptr(gate_prev),
                            _ptr(pos_bias), _dtype_code(kv_cur), B, T, d, m, int(t0), kind,
                            ctypes.byref(st), _stream(stream))
    _check(s, "v4attn_compress")
    return out


def v4attn_compress_nr(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, m, t0, out, nr,
                       stream=None):
    """v4attn_compress with the KV-entry RMSNorm and RoPE of `nr` (NormRope)."""
    lib = load()
    _need_cuda(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias)
    B, T, d = kv_cur.shape
    kind = OUT_KV if isinstance(out, KVCache) else OUT_IDX
    st, ns = out.c_struct(), nr.c_struct()
    s = lib.v4attn_compress_nr(_ptr(kv_cur), _ptr(gate_cur), _ptr(kv_prev), _ptr(gate_prev),
                               _ptr(pos_bias), _dtype_code(kv_cur), B, T, d, m, int(t0), kind,
                               ctypes.byref(st), ctypes.byref(ns), _stream(stream))
    _check(s, "v4attn_compress_nr")
    return out


def _index_topk(name, q_idx, w, keys, pos, m, k, topk, ws, stream):
    lib = load()
    _need_cuda(q_idx, w, pos)
    B, Q, H, d = q_idx.shape
    if topk is None:
        topk = torch.empty(B, Q, k, dtype=torch.int32, device=q_idx.device)
    nbytes = v4attn_workspace_bytes(OP_INDEX_TOPK, B, Q, H, d, keys.cap, k, 0)
    ws, wsb = _workspace(ws, nbytes, q_idx.device)
    st = keys.c_struct()
    s = getattr(lib, name)(_ptr(q_idx), _dtype_code(q_idx), _ptr(w), ctypes.byref(st),
                           _ptr(pos), B, Q, H, m, k, _ptr(topk), _ptr(ws), wsb, _stream(stream))
    _check(s, name)
    return topk


def v4attn_index_topk(q_idx, w, keys, pos, m, k, topk=None, ws=None, stream=None):
    return _index_topk("v4attn_index_topk", q_idx, w, keys, pos, m, k, topk, ws, stream)


def v4attn_index_topk_noalloc(q_idx, w, keys, pos, m, k, topk, stream=None):
    """v4attn_index_topk on the library's fixed device scratch: the caller
    passes the output `topk` (int32 [B][Q][k]); nothing is allocated."""
    lib = load()
    _need_cuda(q_idx, w, pos, topk)
    B, Q, H, d = q_idx.shape
    st = keys.c_struct()
    s = lib.v4attn_index_topk_noalloc(_ptr(q_idx), _dtype_code(q_idx), _ptr(w), ctypes.byref(st),
                                      _ptr(pos), B, Q, H, m, k, _ptr(topk), _stream(stream))
    _check(s, "v4attn_index_topk_noalloc")
    return topk


def v4attn_index_topk_bf16(q_idx, w, keys, pos, m, k, topk=None, ws=None, stream=None):
    """The BF16-score selector variant (same arguments as v4attn_index_topk)."""
    return _index_topk("v4attn_index_topk_bf16", q_idx, w, keys, pos, m, k, topk, ws, stream)


def _out(q, out, out_dtype):
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    return out


def v4attn_csa_attend(q, comp, topk, win, n_win, pos, sink, sm_scale, out=None,
                      out_dtype=torch.bfloat16, ws=None, stream=None):
    lib = load()
    _need_cuda(q, topk, pos, sink)
    B, Q, H, D = q.shape
    k = topk.shape[-1]
    out = _out(q, out, out_dtype)
    nbytes = v4attn_workspace_bytes(OP_CSA_ATTEND, B, Q, H, D, comp.cap, k, n_win)
    ws, wsb = _workspace(ws, nbytes, q.device)
    cs, wst = comp.c_struct(), win.c_struct()
    s = lib.v4attn_csa_attend(_ptr(q), _dtype_code(q), ctypes.byref(cs), _ptr(topk), k,
                              ctypes.byref(wst), n_win, _ptr(pos), _ptr(sink), float(sm_scale),
                              B, Q, H, _ptr(out), _dtype_code(out), _ptr(ws), wsb, _stream(stream))
    _check(s, "v4attn_csa_attend")
    return out


def v4attn_csa_index_attend(q_idx, w, keys, m, k, q, comp, win, n_win, pos, sink, sm_scale,
                            topk=None, out=None, out_dtype=torch.bfloat16, ws_index=None,
                            ws_attend=None, stream=None):
    """v4attn_index_topk followed by v4attn_csa_attend in one call (the
    selector's ordering step inside the attention kernel); returns
    (topk, out)."""
    lib = load()
    _need_cuda(q_idx, w, q, pos, sink)
    B, Q, H_I, d = q_idx.shape
    H, D = q.shape[2], q.shape[3]
    if topk is None:
        topk = torch.empty(B, Q, k, dtype=torch.int32, device=q.device)
    out = _out(q, out, out_dtype)
    ws_index, wib = _workspace(ws_index, v4attn_workspace_bytes(OP_CSA_INDEX, B, Q, H_I, d,
                                                                keys.cap, k, 0), q.device)
    ws_attend, wab = _workspace(ws_attend, v4attn_workspace_bytes(OP_CSA_ATTEND, B, Q, H, D,
                                                                  comp.cap, k, n_win), q.device)
    ks, cs, wst = keys.c_struct(), comp.c_struct(), win.c_struct()
    s = lib.v4attn_csa_index_attend(_ptr(q_idx), _dtype_code(q_idx), _ptr(w), ctypes.byref(ks),
                                    H_I, m, k, _ptr(topk), _ptr(q), _dtype_code(q),
                                    ctypes.byref(cs), ctypes.byref(wst), n_win, _ptr(pos),
                                    _ptr(sink), float(sm_scale), B, Q, H, _ptr(out),
                                    _dtype_code(out), _ptr(ws_index), wib, _ptr(ws_attend), wab,
                                    _stream(stream))
    _check(s, "v4attn_csa_index_attend")
    return topk, out


def v4attn_hca_attend(q, comp, m, win, n_win, pos, sink, sm_scale, out=None,
                      out_dtype=torch.bfloat16, ws=None, stream=None):
    lib = load()
    _need_cuda(q, pos, sink)
    B, Q, H, D = q.shape
    out = _out(q, out, out_dtype)
    nbytes = v4attn_workspace_bytes(OP_HCA_ATTEND, B, Q, H, D, comp.cap, m, n_win)
    ws, wsb = _workspace(ws, nbytes, q.device)
    cs, wst = comp.c_struct(), win.c_struct()
    s = lib.v4attn_hca_attend(_ptr(q), _dtype_code(q), ctypes.byref(cs), m, ctypes.byref(wst),
                              n_win, _ptr(pos), _ptr(sink), float(sm_scale), B, Q, H,
                              _ptr(out), _dtype_code(out), _ptr(ws), wsb, _stream(stream))
    _check(s, "v4attn_hca_attend")
    return out


def v4attn_csa_attend_nr(q, comp, topk, win, n_win, pos, sink, sm_scale, nr, out=None,
                         out_dtype=torch.bfloat16, ws=None, stream=None):
    """v4attn_csa_attend with the query RMSNorm + RoPE and the output's
    rotation back of `nr` (NormRope)."""
    lib = load()
    _need_cuda(q, topk, pos, sink)
    B, Q, H, D = q.shape
    k = topk.shape[-1]
    out = _out(q, out, out_dtype)
    nbytes = v4attn_workspace_bytes(OP_CSA_ATTEND_NR, B, Q, H, D, comp.cap, k, n_win)
    ws, wsb = _workspace(ws, nbytes, q.device)
    cs, wst, ns = comp.c_struct(), win.c_struct(), nr.c_struct()
    s = lib.v4attn_csa_attend_nr(_ptr(q), _dtype_code(q), ctypes.byref(cs), _ptr(topk), k,
                                 ctypes.byref(wst), n_win, _ptr(pos), _ptr(sink), float(sm_scale),
                                 B, Q, H, _ptr(out), _dtype_code(out), ctypes.byref(ns), _ptr(ws),
                                 wsb, _stream(stream))
    _check(s, "v4attn_csa_attend_nr")
    return out


def v4attn_hca_attend_nr(q, comp, m, win, n_win, pos, sink, sm_scale, nr, out=None,
                         out_dtype=torch.bfloat16, ws=None, stream=None):
    """v4attn_hca_attend with the query RMSNorm + RoPE and the output's
    rotation back of `nr` (NormRope)."""
    lib = load()
    _need_cuda(q, pos, sink)
    B, Q, H, D = q.shape
    out = _out(q, out, out_dtype)
    nbytes = v4attn_workspace_bytes(OP_HCA_ATTEND_NR, B, Q, H, D, comp.cap, m, n_win)
    ws, wsb = _workspace(ws, nbytes, q.device)
    cs, wst, ns = comp.c_struct(), win.c_struct(), nr.c_struct()
    s = lib.v4attn_hca_attend_nr(_ptr(q), _dtype_code(q), ctypes.byref(cs), m, ctypes.byref(wst),
                                 n_win, _ptr(pos), _ptr(sink), float(sm_scale), B, Q, H,
                                 _ptr(out), _dtype_code(out), ctypes.byref(ns), _ptr(ws), wsb,
                                 _stream(stream))
    _check(s, "v4attn_hca_attend_nr")
    return out


# ---------------------------------------------------------------- paged cache

@dataclass
class Pages:
    """[Notes §11] block table of a paged cache: table int32 [B][max_pages]
    (device) naming each sequence's pool pages, page_tokens raw tokens per
    page.  A paged KVCache / IdxCache is the pool: batch axis 1, n_pages * P
    rows, P = page_tokens / m."""
    table: torch.Tensor
    page_tokens: int

    def entries_per_page(self, m):
        return self.page_tokens // m

    def logical_cap(self, m):
        return self.table.shape[1] * self.entries_per_page(m)

    def c_struct(self):
        _need_cuda(self.table)
        if self.table.dtype != torch.int32 or self.table.dim() != 2 or not self.table.is_contiguous():
            raise V4AttnError("page table must be a contiguous int32 [B][max_pages] tensor")
        return _Pages(self.table.data_ptr(), self.table.shape[1], int(self.page_tokens))


def append_state(B, d, device="cuda"):
    """Pooling state of v4attn_append: f32 [B][2][3][d] (no initialisation
    needed: a sequence's first token at slot 0 of a block resets it)."""
    return torch.empty(B, 2, 3, d, dtype=torch.float32, device=device)


def _byref(st):
    return None if st is None else ctypes.byref(st)


def v4attn_compress_paged(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias, m, t0, out, pages,
                          nr=None, stream=None):
    """v4attn_compress (with nr: its _nr form) into the pool pages of `pages`."""
    lib = load()
    _need_cuda(kv_cur, gate_cur, kv_prev, gate_prev, pos_bias)
    B, T, d = kv_cur.shape
    kind = OUT_KV if isinstance(out, KVCache) else OUT_IDX
    st, ps = out.c_struct(), pages.c_struct()
    ns = None if nr is None else nr.c_struct()
    s = lib.v4attn_compress_paged(_ptr(kv_cur), _ptr(gate_cur), _ptr(kv_prev), _ptr(gate_prev),
                                  _ptr(pos_bias), _dtype_code(kv_cur), B, T, d, m, int(t0), kind,
                                  ctypes.byref(st), ctypes.byref(ps), _byref(ns), _stream(stream))
    _check(s, "v4attn_compress_paged")
    return out


def v4attn_append(kv_cur, gate_cur, kv_prev, gate_prev, state, pos, pos_bias, m, out, pages=None,
                  nr=None, stream=None):
    """One decode step of the compressor: token rows [B][d] at positions pos
    [B] fold into `state` (append_state, or None for m = 1 without overlap);
    completed blocks go to `out` (None: the state alone is updated)."""
    lib = load()
    _need_cuda(kv_cur, gate_cur, kv_prev, gate_prev, state, pos, pos_bias)
    B, d = kv_cur.shape
    if state is not None and (state.dtype != torch.float32 or state.numel() < B * 6 * d):
        raise V4AttnError("append state must be f32 [B][2][3][d]")
    kind = OUT_KV if isinstance(out, KVCache) else OUT_IDX
    st = None if out is None else out.c_struct()
    ps = None if pages is None else pages.c_struct()
    ns = None if nr is None else nr.c_struct()
    s = lib.v4attn_append(_ptr(kv_cur), _ptr(gate_cur), _ptr(kv_prev), _ptr(gate_prev),
                          _ptr(state), _ptr(pos), _ptr(pos_bias), _dtype_code(kv_cur), B, d, m,
                          kind, _byref(st), _byref(ps), _byref(ns), _stream(stream))
    _check(s, "v4attn_append")
    return out


def v4attn_append_batch(calls, stream=None):
    """Several v4attn_append calls in one launch.  `calls`: dicts with the
    keyword arguments of v4attn_append (kv_cur, gate_cur, kv_prev, gate_prev,
    state, pos, pos_bias, m, out, pages, nr); no two may write the same state
    or cache rows."""
    lib = load()
    keep = []                                   # host structs the call points to

    def ref(st):
        if st is None:
            return None
        keep.append(st)
        return ctypes.cast(ctypes.pointer(st), ctypes.c_void_p)

    arr = (_Append * max(1, len(calls)))()
    for j, c in enumerate(calls):
        kv = c["kv_cur"]
        _need_cuda(kv, c.get("gate_cur"), c.get("kv_prev"), c.get("gate_prev"), c.get("state"),
                   c["pos"], c.get("pos_bias"))
        B, d = kv.shape
        out = c.get("out")
        kind = OUT_KV if isinstance(out, KVCache) else OUT_IDX
        pg, nr = c.get("pages"), c.get("nr")
        arr[j] = _Append(_ptr(kv), _ptr(c.get("gate_cur")), _ptr(c.get("kv_prev")),
                         _ptr(c.get("gate_prev")), _ptr(c.get("state")), _ptr(c["pos"]),
                         _ptr(c.get("pos_bias")), ref(None if out is None else out.c_struct()),
                         ref(None if pg is None else pg.c_struct()),
                         ref(None if nr is None else nr.c_struct()), _dtype_code(kv), B, d,
                         int(c["m"]), kind, 0)
    s = lib.v4attn_append_batch(len(calls), arr, _stream(stream))
    _check(s, "v4attn_append_batch")


def v4attn_index_topk_paged(q_idx, w, keys, pages, pos, m, k, score_bf16=False, topk=None,
                            ws=None, stream=None):
    lib = load()
    _need_cuda(q_idx, w, pos)
    B, Q, H, d = q_idx.shape
    if topk is None:
        topk = torch.empty(B, Q, k, dtype=torch.int32, device=q_idx.device)
    nbytes = v4attn_workspace_bytes(OP_INDEX_TOPK, B, Q, H, d, pages.logical_cap(m), k, 0)
    ws, wsb = _workspace(ws, nbytes, q_idx.device)
    st, ps = keys.c_struct(), pages.c_struct()
    s = lib.v4attn_index_topk_paged(_ptr(q_idx), _dtype_code(q_idx), _ptr(w), ctypes.byref(st),
                                    ctypes.byref(ps), _ptr(pos), B, Q, H, m, k,
                                    1 if score_bf16 else 0, _ptr(topk), _ptr(ws), wsb,
                                    _stream(stream))
    _check(s, "v4attn_index_topk_paged")
    return topk


def v4attn_csa_attend_paged(q, comp, pages, m, topk, win, n_win, pos, sink, sm_scale, nr=None,
                            out=None, out_dtype=torch.bfloat16, ws=None, stream=None):
    lib = load()
    _need_cuda(q, topk, pos, sink)
    B, Q, H, D = q.shape
    k = topk.shape[-1]
    out = _out(q, out, out_dtype)
    op = OP_CSA_ATTEND if nr is None else OP_CSA_ATTEND_NR
    nbytes = v4attn_workspace_bytes(op, B, Q, H, D, pages.logical_cap(m), k, n_win)
    ws, wsb = _workspace(ws, nbytes, q.device)
    cs, wst, ps = comp.c_struct(), win.c_struct(), pages.c_struct()
    ns = None if nr is None else nr.c_struct()
    s = lib.v4attn_csa_attend_paged(_ptr(q), _dtype_code(q), ctypes.byref(cs), ctypes.byref(ps), m,
                                    _ptr(topk), k, ctypes.byref(wst), n_win, _ptr(pos), _ptr(sink),
                                    float(sm_scale), B, Q, H, _ptr(out), _dtype_code(out),
                                    _byref(ns), _ptr(ws), wsb, _stream(stream))
    _check(s, "v4attn_csa_attend_paged")
    return out


def v4attn_hca_attend_paged(q, comp, pages, m, win, n_win, pos, sink, sm_scale, nr=None, out=None,
                            out_dtype=torch.bfloat16, ws=None, stream=None):
    lib = load()
    _need_cuda(q, pos, sink)
    B, Q, H, D = q.shape
    out = _out(q, out, out_dtype)
    op = OP_HCA_ATTEND if nr is None else OP_HCA_ATTEND_NR
    nbytes = v4attn_workspace_bytes(op, B, Q, H, D, pages.logical_cap(m), m, n_win)
    ws, wsb = _workspace(ws, nbytes, q.device)
    cs, wst, ps = comp.c_struct(), win.c_struct(), pages.c_struct()
    ns = None if nr is None else nr.c_struct()
    s = lib.v4attn_hca_attend_paged(_ptr(q), _dtype_code(q), ctypes.byref(cs), ctypes.byref(ps), m,
                                    ctypes.byref(wst), n_win, _ptr(pos), _ptr(sink),
                                    float(sm_scale), B, Q, H, _ptr(out), _dtype_code(out),
                                    _byref(ns), _ptr(ws), wsb, _stream(stream))
    _check(s, "v4attn_hca_attend_paged")
    return out
