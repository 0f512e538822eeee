// Kernel argument blocks and launchers (host-visible; no torch, no ABI types).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace v4a {

// Paged classical cache ([Notes §11]): logical row r of sequence b lives at
// pool row tab[b * tab_ld + (r >> psh)] * 2^psh + (r & (2^psh - 1)).  Page
// ids are clamped into [0, n_pages) on the device, so no table content can
// address outside the pool.  tab == null: the contiguous [B][cap] layout.
struct Pages {
  const int32_t* tab;
  int tab_ld;                // table row length (pages per sequence)
  int psh;                   // log2 of the entries per page
  int64_t n_pages;           // pages in the pool
};

__device__ __forceinline__ int64_t page_row(const Pages& pg, int b, int64_t r) {
  int64_t p = pg.tab[(int64_t)b * pg.tab_ld + (r >> pg.psh)];
  p = p < 0 ? 0 : (p >= pg.n_pages ? pg.n_pages - 1 : p);
  return (p << pg.psh) | (r & (((int64_t)1 << pg.psh) - 1));
}

// ---------------------------------------------------------------- compress
struct CompressArgs {
  const void* kv_cur;
  const void* gate_cur;      // may be null (zero gates)
  const void* kv_prev;       // null = no overlap
  const void* gate_prev;     // may be null (zero gates) when kv_prev is set
  const float* bias;         // may be null (zero bias); [slots][d]
  int in_bf16;
  int B, T, d, m;
  int64_t t0;
  int out_kind;              // 0 = KV entries, 1 = indexer keys
  int out_fmt;               // 0 = f32, 2 = FP8+BF16 RoPE (KV) / 3 = MXFP4 (keys)
  int d_nope;                // KV: split point
  int64_t cap;
  void* o_a;                 // KV: nope (f32 | u8 e4m3);  keys: codes (f32 | u8 packed)
  void* o_b;                 // KV: rope (f32 | bf16);     keys: e8m0 scales
  float* o_scale;            // KV FP8: per-entry scale
  // KV-entry RMSNorm / RoPE before the store (null: off)
  const float* nr_gamma;     // [d]
  const float* nr_inv;       // [d_rope / 2] inverse frequencies
  float nr_eps;
  Pages pg;                  // paged output: row = page_row(block), no ring
  // decode-time append (apos non-null): one token per sequence, kv_* / gate_*
  // are [B][d]; state [B][2][3][d] holds the running pooling of each sequence
  const int64_t* apos;       // [B] the token's position (< 0: sequence idle)
  float* state;              // null only for m == 1 without overlap
  int no_store;              // 1: update the state only (no output cache)
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t st);
// up to kMaxAppend decode-time appends in one launch
constexpr int kMaxAppend = 8;
struct AppendBatch {
  CompressArgs c[kMaxAppend];
  int n;
};
hipError_t launch_append_batch(const AppendBatch& ab, hipStream_t st);

// ---------------------------------------------------------------- indexer + top-k
struct IndexArgs {
  const void* q;             // [R][H][d]
  int q_bf16;
  const float* w;            // [R][H]
  const void* codes;         // keys: f32 [B][cap][d] | u8 [B][cap][d/2]
  const uint8_t* kscales;    // e8m0 [B][cap][d/32] (MXFP4)
  int key_mx;
  int64_t cap;
  int d;
  const int64_t* pos;        // [R]
  int B, Q, H, m, k;
  int32_t* topk;             // [R][k]
  int score_bf16;            // 1: scores are cut to bf16 (RNE) and ranked as
                             // such; the workspace's score rows hold bf16
  // scan plan (one-query-per-workgroup FP4 scan)
  int score_iters;           // 1024-block iterations per scan workgroup
  int score_wgs;             // scan workgroups per query
  int hp_ld;                 // > 0 (= score_wgs): the scan writes per-workgroup
                             // first-digit histograms and zeroes the filter
                             // counters itself (no prep kernel)
  // workspace regions
  uint8_t* qmx;              // [R][H][d/2]
  uint8_t* qsc;              // [R][H][d/32]
  float* scores;             // [R][sc_ld] fp32, or bf16 (score_bf16) in the same space
  int64_t sc_ld;             // score row stride (cap rounded up to 64)
  uint32_t* hist;            // [R][256] first-digit histogram (key bits 31..24)
  uint32_t* hist2;           // [R][2048] second digit (key bits 23..13) within the first
  uint32_t* ctr;             // [R][8] candidate count, threshold digits
  uint64_t* cand;            // [R][16384] candidate keys (score key : inverted id)
  uint32_t* chunk;           // [R][n_chunks] per filter chunk: ids above the candidates
  uint16_t* hparts;          // [R][hp_ld][256] per-scan-workgroup first-digit counts
  float* samp;               // [R][samp_ld] sample-tile scores (query-tiled scans), or null
  int64_t samp_ld;
  int fb_only;               // 1: the full-score kernels take only the rows handed over
  uint32_t* fbl;             // [1 + R]: count, then the rows handed over (sampled path)
  Pages pg;                  // paged keys (MXFP4 only; >= 128 keys per page)
  // selection fused with the CSA attention (null: the emit kernel writes
  // topk): k_filter2 writes, per chunk, the selection keys of every id at
  // or above the candidates' bin in id order, and no emit kernel runs
  uint64_t* elist;           // [R][n_chunks][4096]
  uint32_t* elen;            // [R][n_chunks] list lengths
};
// fused = 1: with the per-chunk lists of the fused selection
size_t index_workspace_bytes(int B, int Q, int H, int d, int64_t cap, int key_mx, int fused = 0);
void index_carve(IndexArgs& a, void* ws, int fused = 0);
// The call takes the three-filter selection (k_filter1, k_filter2, k_emit)
// for every row, with at most kSelMaxChunks filter chunks per row, so that
// its emit step can move into the CSA attention.
bool index_filter_path(const IndexArgs& a);
// `ev` (may be null): a start / stop event pair recorded around the call's
// dominant kernel (hipExtLaunchKernelGGL), for kernel-level timing.
struct KernelEvents {
  hipEvent_t start, stop;
};
hipError_t launch_index_topk(const IndexArgs& a, hipStream_t st, const KernelEvents* ev);
// Fixed device scratch of the allocation-free index call: its size, and its
// device address on the current device (looked up once per device).
constexpr size_t kIndexScratchBytes = (size_t)32 << 20;
hipError_t index_scratch(void** ptr);

// ---------------------------------------------------------------- attend
struct AttendArgs {
  const void* q;             // [R][H][D]
  int q_bf16;
  const uint8_t* c_nope;     // compressed entries (typed as bytes; f32 in fp32 mode)
  const uint16_t* c_rope;
  const float* c_scale;
  int64_t c_cap;
  const uint8_t* w_nope;     // window ring
  const uint16_t* w_rope;
  const float* w_scale;
  int64_t w_cap;
  int csa;                   // 1: compressed part = the k top-k slots; 0: HCA
  const int32_t* topk;       // CSA: [R][k] (may be null when k == 0)
  int k;
  int m;                     // HCA compression rate
  int n_win;
  const int64_t* pos;
  const float* sink;         // [H] or null
  float sm_scale;
  int B, Q, H, d_nope, d_rope;
  void* out;
  int out_bf16;
  int fp8;                   // 1 = FP8 MFMA path, 0 = fp32 VALU path
  int f32_heads;             // heads per workgroup on the fp32 path
  int n_split, split_size;   // entry-list split (fixed by the per-query shape)
  int part_bf16;             // split partials stored in bf16 (FP8 path) or fp32
  void* part_o;              // [R][n_split][H][D] O / l
  float* part_ml;            // [R][n_split][H][2] (max, denominator)
  // query RMSNorm / RoPE in the attention prologue and the output's rotation
  // back (k_attend_fp8_nr when either is set)
  const float* nr_gamma;     // [D] or null
  const float* nr_inv;       // [d_rope / 2] or null
  float nr_eps;
  Pages c_pg;                // paged compressed cache (FP8 path only)
  // fused selection (FP8 CSA only; sel_ctr null: the ids are read from
  // topk): each workgroup derives the ids of its split's top-k slots from
  // the selector's filter results (IndexArgs ctr / cand / elist / elen /
  // scores of the same rows) and head group 0 writes them to sel_topk
  const uint32_t* sel_ctr;
  const uint64_t* sel_cand;
  const uint64_t* sel_elist;
  const uint32_t* sel_elen;
  const float* sel_scores;
  int64_t sel_sc_ld;
  int64_t sel_cap;           // the indexer keys' capacity
  int sel_m;                 // their compression rate
  int32_t* sel_topk;         // [R][k]
};
// The fused selection handles at most this many filter chunks per row and
// splits of at most 256 entries.
constexpr int kSelMaxChunks = 1024;
void attend_plan(AttendArgs& a, int64_t n_entries_max);
size_t attend_workspace_bytes(const AttendArgs& a);
void attend_carve(AttendArgs& a, void* ws);
hipError_t launch_attend(const AttendArgs& a, hipStream_t st, const KernelEvents* ev);

}  // namespace v4a
