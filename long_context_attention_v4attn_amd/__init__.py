"""MI355X (gfx950) CSA / HCA hybrid compressed attention.

The compute lives in ``libv4attn.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/v4attn.h``); this package is a thin ctypes binding
that marshals torch tensors (device memory and streams) into those calls.
There is no CPU or PyTorch fallback: every call fails loudly when the library
is not built or no GPU is present.
"""

from .binding import (  # noqa: F401
    F32, BF16, KV_FP8_BF16ROPE, IDX_MXFP4, OP_INDEX_TOPK, OP_CSA_ATTEND, OP_HCA_ATTEND,
    KVCache, IdxCache, V4AttnError, load, library_path,
    v4attn_compress, v4attn_index_topk, v4attn_index_topk_bf16, v4attn_index_topk_noalloc,
    v4attn_csa_attend, v4attn_csa_index_attend, OP_CSA_INDEX,
    v4attn_hca_attend, NormRope, OP_CSA_ATTEND_NR, OP_HCA_ATTEND_NR, v4attn_compress_nr,
    v4attn_csa_attend_nr, v4attn_hca_attend_nr,
    Pages, append_state, v4attn_compress_paged, v4attn_append, v4attn_append_batch, v4attn_index_topk_paged,
    v4attn_csa_attend_paged, v4attn_hca_attend_paged,
    v4attn_workspace_bytes, v4attn_status_str, v4attn_time_next_kernel,
)
