// Lightning indexer and top-k selector.
//
// Method: [Notes §7] index score I_{t,s} = sum_h w_{t,h} ReLU(q_{t,h} . K_s)
// over the compressed blocks visible to query t, then Top-k over s;
// [Notes §9] the indexer's QK path runs in FP4 (keys and queries MXFP4), and
// the selector ranks fp32 scores -- or, in the BF16-score variant of the same
// section, the scores rounded to bf16 (which the score rows then hold).
//
// Pipeline of one v4attn_index_topk call, one query per sequence (decode:
// four launches with 16 index heads, five otherwise):
//   k_prep       (other head counts) query heads -> MXFP4 (e2m1 codes + e8m0
//                scale per 32); zero the per-query histogram and counters.
//   k_score_mx   FP4 scan: one v_mfma_scale_f32_16x16x128_f8f6f4 per
//                (16 index heads, 16 blocks): M = heads, N = blocks, K = 128
//                dims; the e8m0 scales feed the MFMA's scale operands, so the
//                per-head dots are exact.  fp32 epilogue: ReLU, head weight,
//                sum over heads (in-lane over 4 heads, then across the four
//                lane groups).  A wave streams 256 blocks per iteration (16 KB
//                of keys in coalesced 1 KB loads); the next iteration's loads
//                are in flight while the current one computes.  The
//                workgroup histograms the first radix digit (key bits
//                31..24) of its scores' order-preserving keys in LDS and
//                writes it as one partial row (16 index heads: it also
//                quantises its query heads and zeroes the counters, so no
//                kernel runs before it) or adds it to the query's global
//                histogram.
//   k_score_f32  fp32 VALU variant for unquantised keys (same histogram).
//   k_filter1    per query, many workgroups (4096 scores each): the
//                histogram gives the bin b1 (key bits 31..24) that holds the
//                k-th largest score; ids in b1 are histogrammed on bits 23..13.
//   k_filter2    same split: the second histogram gives the bin b2; each
//                workgroup counts its ids above (b1, b2) and appends the ids
//                in (b1, b2) as candidates.
//   k_emit       same split: every workgroup resolves the exact threshold T
//                among the (few) candidates (radix select on the 64-bit key =
//                score key : inverted id, so ties go to the lower id), then
//                writes every id of its chunk whose key is >= T at the
//                chunk's offset plus its rank within the chunk: the k ids
//                come out ascending with no sort; the tail is -1.  No
//                workgroup waits for another, and the output is
//                deterministic.
// In the fused CSA call (v4attn_csa_index_attend) k_filter2 also writes each
// chunk's selection keys at or above the candidates' bin in id order, and
// the attention kernel takes the emit step (no k_emit launch).
// Query-tiled scans (many queries per sequence: prefill chunks) take the
// sampled-threshold selection described at k_thresh below.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace v4a {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Sampled-threshold selection of query-tiled scans (prefill chunks): the
// sample is every 16th tile of 16 blocks (blocks 256 j .. 256 j + 15).
__host__ __device__ inline int64_t n_sampled(int64_t nv) {
  return (nv >> 8) * 16 + ((nv & 255) < 16 ? (nv & 255) : 16);
}
__host__ __device__ inline int64_t samp_ld(int64_t cap) { return (n_sampled(cap) + 63) / 64 * 64; }
constexpr int kFbRows = 32;                // rows the full-score filters take at a time
constexpr int kThrPer = 68;                // sample keys per k_thresh thread (n_sampled <= 17408)
constexpr int kPfBmWords = 8448;           // its id bitmap in LDS: up to 270336 blocks
// The query-tiled scan (16 index heads, MXFP4 keys, >= 8 queries per
// sequence) takes the sampled-threshold path when the id bitmap fits.
__host__ __device__ inline bool pf_sampled(int64_t cap, int H, int Q, int key_mx) {
  return key_mx && H == 16 && Q >= 8 && cap <= (int64_t)kPfBmWords * 32;
}

constexpr int kWaveTiles = 8;              // 8 tiles x 16 blocks per wave and iteration
constexpr int kScanWaves = 4;              // waves per scan workgroup
constexpr int kIterBlocks = kScanWaves * kWaveTiles * 16;   // 512 blocks per workgroup iteration
constexpr int kQT = 8;                     // queries per workgroup of the query-tiled scan
constexpr int kMaxParts = 128;             // widest partial-histogram row
constexpr int kMaxIters = 32;              // iterations per scan workgroup (<= 16384 blocks)

// Plan of the one-query-per-workgroup FP4 scan: about 512 workgroups of 4
// waves in all (two per CU), each walking `iters` iterations of kIterBlocks
// blocks.  With 16
// index heads, when every workgroup's count fits 16 bits and there are at
// most kMaxParts workgroups per query, the workgroups write partial
// first-digit histograms (hp_ld = workgroups per query, else 0).
struct ScanPlan {
  int iters, wgs, hp_ld;
};

static ScanPlan scan_plan(int64_t cap, int64_t R, int H, int Q, int key_mx) {
  ScanPlan p{0, 0, 0};
  if (!key_mx || (H == 16 && Q >= kQT)) return p;
  const int64_t it_total = (cap + kIterBlocks - 1) / kIterBlocks;
  int64_t iters = (it_total * R + 511) / 512;
  if (iters < 1) iters = 1;
  if (iters > it_total) iters = it_total;
  if (iters > kMaxIters) iters = kMaxIters;
  p.iters = (int)iters;
  p.wgs = (int)((it_total + iters - 1) / iters);
  if (H == 16 && iters * kIterBlocks <= 65535 && p.wgs <= kMaxParts) p.hp_ld = p.wgs;
  return p;
}

size_t index_workspace_bytes(int B, int Q, int H, int d, int64_t cap, int key_mx, int fused) {
  const size_t R = (size_t)B * Q;
  const ScanPlan sp = scan_plan(cap, (int64_t)R, H, Q, key_mx);
  size_t n = align256(R * kBins1 * (size_t)sp.hp_ld * sizeof(uint16_t));
  if (key_mx) n += align256(R * H * (d / 2)) + align256(R * H * (d / 32));
  n += align256(R * (size_t)score_ld(cap) * sizeof(float));
  n += align256(R * kBins1 * sizeof(uint32_t)) + align256(R * kBins2 * sizeof(uint32_t));
  n += align256(R * kCtr * sizeof(uint32_t));
  n += align256(R * kCandCap * sizeof(uint64_t));
  n += align256(R * (size_t)n_chunks(cap) * sizeof(uint32_t));
  if (pf_sampled(cap, H, Q, key_mx))
    n += align256(R * (size_t)samp_ld(cap) * sizeof(float)) + align256((R + 1) * sizeof(uint32_t));
  if (fused)
    n += align256(R * (size_t)n_chunks(cap) * kFilterChunk * sizeof(uint64_t)) +
         align256(R * (size_t)n_chunks(cap) * sizeof(uint32_t));
  return n;
}

bool index_filter_path(const IndexArgs& a) {
  return !pf_sampled(a.cap, a.H, a.Q, a.key_mx) && !a.score_bf16 &&
         n_chunks(a.cap) <= kSelMaxChunks;
}

void index_carve(IndexArgs& a, void* ws, int fused) {
  const size_t R = (size_t)a.B * a.Q;
  const ScanPlan sp = scan_plan(a.cap, (int64_t)R, a.H, a.Q, a.key_mx);
  a.score_iters = sp.iters;
  a.score_wgs = sp.wgs;
  // the scan's own query quantisation loads 16-byte vectors
  a.hp_ld = ((uintptr_t)a.q & 15) ? 0 : sp.hp_ld;
  char* p = (char*)ws;
  a.hparts = (uint16_t*)p;
  p += align256(R * kBins1 * (size_t)sp.hp_ld * sizeof(uint16_t));
  a.qmx = nullptr;
  a.qsc = nullptr;
  if (a.key_mx) {
    a.qmx = (uint8_t*)p;
    p += align256(R * a.H * (a.d / 2));
    a.qsc = (uint8_t*)p;
    p += align256(R * a.H * (a.d / 32));
  }
  a.sc_ld = score_ld(a.cap);
  a.scores = (float*)p;
  p += align256(R * (size_t)a.sc_ld * sizeof(float));
  a.hist = (uint32_t*)p;
  p += align256(R * kBins1 * sizeof(uint32_t));
  a.hist2 = (uint32_t*)p;
  p += align256(R * kBins2 * sizeof(uint32_t));
  a.ctr = (uint32_t*)p;
  p += align256(R * kCtr * sizeof(uint32_t));
  a.cand = (uint64_t*)p;
  p += align256(R * kCandCap * sizeof(uint64_t));
  a.chunk = (uint32_t*)p;
  p += align256(R * (size_t)n_chunks(a.cap) * sizeof(uint32_t));
  a.samp = nullptr;
  a.samp_ld = samp_ld(a.cap);
  a.fb_only = 0;
  a.fbl = nullptr;
  if (pf_sampled(a.cap, a.H, a.Q, a.key_mx)) {
    a.samp = (float*)p;
    p += align256(R * (size_t)a.samp_ld * sizeof(float));
    a.fbl = (uint32_t*)p;
    p += align256((R + 1) * sizeof(uint32_t));
  }
  a.elist = nullptr;
  a.elen = nullptr;
  if (fused) {
    a.elist = (uint64_t*)p;
    p += align256(R * (size_t)n_chunks(a.cap) * kFilterChunk * sizeof(uint64_t));
    a.elen = (uint32_t*)p;
  }
}

// The selector's score precision.  fp32, or the bf16 variant ([Notes §9]:
// index scores cut from FP32 to BF16 in the top-k selector): the fp32 score
// rounded to the nearest bf16 (ties to even, v_cvt_pk_bf16_f32) is what is
// ranked and what the score rows hold (its 16 high bits).  A bf16 value's
// key has its low 16 bits zero, so the radix digits below work unchanged.
__device__ __forceinline__ float ranked(float s, int bf16) {
  return bf16 ? (float)(__bf16)s : s;
}

// The smallest score whose key is >= k: for every non-NaN score s,
// score_key(s) >= k exactly when s >= key_floor(k) (a float compare in place
// of the key; keys below that of -inf admit every score, keys above that of
// +inf none).
__device__ __forceinline__ float key_floor(uint32_t k) {
  if (k <= 0x007FFFFFu) return -INFINITY;
  if (k > 0xFF800000u) return __uint_as_float(0x7FC00000u);   // NaN: no score compares >=
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ void put_score(const IndexArgs& a, size_t i, float r) {
  if (a.score_bf16)
    ((uint16_t*)a.scores)[i] = (uint16_t)(__float_as_uint(r) >> 16);
  else
    a.scores[i] = r;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// ---------------------------------------------------------------- prep
__global__ void __launch_bounds__(256) k_prep(IndexArgs a) {
  const int R = a.B * a.Q;
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nthr = (size_t)gridDim.x * blockDim.x;
  for (size_t i = tid; i < (size_t)R * kBins1; i += nthr) a.hist[i] = 0u;
  for (size_t i = tid; i < (size_t)R * kBins2; i += nthr) a.hist2[i] = 0u;
  for (size_t i = tid; i < (size_t)R * kCtr; i += nthr) a.ctr[i] = 0u;
  if (a.fbl && tid == 0) a.fbl[0] = 0u;    // rows handed to the full-score path
  if (!a.key_mx) return;
  // one wave per (row, head): 128 elements, 2 per lane; a group of 32 is 16 lanes
  const int lane = threadIdx.x & 63;
  for (size_t wave = tid >> 6; wave < (size_t)R * a.H; wave += nthr >> 6) {
    const size_t base = wave * a.d;
    float x0 = load_as_f32(a.q, a.q_bf16, base + 2 * lane);
    float x1 = load_as_f32(a.q, a.q_bf16, base + 2 * lane + 1);
    float am = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    int e = mx_exponent(am);
    float inv = ldexpf(1.0f, -e);
    uint32_t c0 = am > 0.f ? enc_e2m1(x0 * inv) : 0u;
    uint32_t c1 = am > 0.f ? enc_e2m1(x1 * inv) : 0u;
    a.qmx[wave * (a.d / 2) + lane] = (uint8_t)(c0 | (c1 << 4));
    if ((lane & 15) == 0) a.qsc[wave * (a.d / 32) + (lane >> 4)] = (uint8_t)(e + 127);
  }
}

// LDS histogram of nb bins flushed to the query's global histogram
// (non-empty bins only).
__device__ __forceinline__ void hist_flush(uint32_t* lh, uint32_t* gh, int nb) {
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += blockDim.x) {
    uint32_t c = lh[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// ---------------------------------------------------------------- FP4 scan

// x + y after swapping x's lanes 32..63 with y's lanes 0..31: lanes 0..31
// hold x summed over lane groups {0, 2} resp. {1, 3}, lanes 32..63 the same
// for y.
// (The optimiser of this toolchain folds the two results of a swap into one
// value when both feed the same add; the empty asm statement -- no
// instruction, it only marks both registers as read and written -- keeps
// them apart.)
__device__ __forceinline__ float swap_add32(float x, float y) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, y), false, false);
  uint32_t lo = r[0], hi = r[1];
  __asm__ volatile("" : "+v"(lo), "+v"(hi));
  return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// The same within each half: swaps x's lanes 16..31 (48..63) with y's lanes
// 0..15 (32..47).
__device__ __forceinline__ float swap_add16(float x, float y) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, y), false, false);
  uint32_t lo = r[0], hi = r[1];
  __asm__ volatile("" : "+v"(lo), "+v"(hi));
  return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// A wave's key tiles of one iteration: per tile the lane's 16 code bytes;
// the e8m0 scales as one dword (the 4 group scales of a block) per four
// tiles -- lane group g holds the dword of block 16 (t4 + g) + li -- which
// the scoring hands to the right lanes with ds_bpermute.  (A wave keeps its
// loads in flight under the 63 the load counter tracks.)
struct KeyTiles {
  u32x4 v[kWaveTiles];
  uint32_t sd[kWaveTiles / 4];
};

// The wave's key tiles of one iteration: tile t = blocks blk0 + 16t + li.
// The addresses do not depend on the query's visible count (blocks past the
// cache end read its last block), so the loads go out before that count is
// known; blocks past the visible count are dropped when the scores are
// stored.  Away from the cache end (the uniform common case) every load is
// one base address plus an immediate offset.
// Paged keys: a page holds >= 128 keys and blk0 is a multiple of 128, so the
// wave's blocks are one contiguous run of pool rows (past the cache end the
// run of the last 128 blocks stands in).
// prow >= 0: that pool row, looked up in advance (paged); -1: look it up here.
__device__ __forceinline__ int64_t paged_run(const Pages& pg, int b, int64_t blk0, int64_t cap) {
  return page_row(pg, b, blk0 < cap ? blk0 : cap - kWaveTiles * 16);
}

__device__ __forceinline__ void load_keys(const uint8_t* kc, const uint8_t* ks, int64_t blk0,
                                          int64_t cap, const Pages& pg, int b, int g, int li,
                                          KeyTiles& kt, int64_t prow = -1) {
  const bool paged = pg.tab != nullptr;
  if (paged || blk0 + kWaveTiles * 16 <= cap) {
    const int64_t r0 = paged ? (prow >= 0 ? prow : paged_run(pg, b, blk0, cap)) : blk0;
    const uint8_t* cp = kc + (r0 + li) * 64 + g * 16;
    const uint32_t* sp = (const uint32_t*)(ks + (r0 + 16 * g + li) * 4);
#pragma unroll
    for (int t = 0; t < kWaveTiles; t++)
      kt.v[t] = __builtin_nontemporal_load((const u32x4*)(cp + t * 1024));
#pragma unroll
    for (int q = 0; q < kWaveTiles / 4; q++) kt.sd[q] = sp[q * 64];
  } else {
#pragma unroll
    for (int t = 0; t < kWaveTiles; t++) {
      int64_t blk = blk0 + t * 16 + li;
      blk = blk < cap ? blk : cap - 1;
      kt.v[t] = __builtin_nontemporal_load((const u32x4*)(kc + blk * 64 + g * 16));
    }
#pragma unroll
    for (int q = 0; q < kWaveTiles / 4; q++) {
      int64_t blk = blk0 + 16 * (4 * q + g) + li;
      blk = blk < cap ? blk : cap - 1;
      kt.sd[q] = *(const uint32_t*)(ks + blk * 4);
    }
  }
}

// MXFP4 fragment of the lane's query head, in two steps so that the loads
// can go out long before the arithmetic: load_q_frag fetches elements
// 32g .. 32g+31 of head h (bf16: 64 bytes, f32: 128 bytes); quantize_q_frag
// encodes them as 16 bytes of e2m1 codes (element 2j in the low nibble of
// byte j) and the group's e8m0 exponent -- the encoding the prep kernel
// writes (the group's 32 elements are all in this lane).
struct QRaw {
  u32x4 v[8];
};

__device__ __forceinline__ void load_q_frag(const IndexArgs& a, int row, int h, int g, QRaw& r) {
  const size_t base = ((size_t)row * a.H + h) * a.d + g * 32;
  if (a.q_bf16) {
    const u32x4* p = (const u32x4*)((const uint16_t*)a.q + base);
#pragma unroll
    for (int i = 0; i < 4; i++) r.v[i] = p[i];
  } else {
    const u32x4* p = (const u32x4*)((const float*)a.q + base);
#pragma unroll
    for (int i = 0; i < 8; i++) r.v[i] = p[i];
  }
}

__device__ __forceinline__ void quantize_q_frag(const IndexArgs& a, const QRaw& r, i32x8* qa,
                                                int* qs) {
  float x[32];
  if (a.q_bf16) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        x[8 * i + 2 * j] = bf16_bits_to_f32(r.v[i][j] & 0xFFFFu);
        x[8 * i + 2 * j + 1] = bf16_bits_to_f32(r.v[i][j] >> 16);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) x[4 * i + j] = __uint_as_float(r.v[i][j]);
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) am = fmaxf(am, fabsf(x[i]));
  const int e = mx_exponent(am);
  const float inv = ldexpf(1.0f, -e);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const uint32_t c0 = am > 0.f ? enc_e2m1(x[2 * j] * inv) : 0u;
    const uint32_t c1 = am > 0.f ? enc_e2m1(x[2 * j + 1] * inv) : 0u;
    w[j / 4] |= (c0 | (c1 << 4)) << (8 * (j % 4));
  }
  *qa = (i32x8){(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
  *qs = e + 127;
}

// Scores of the wave's kWaveTiles tiles, four tiles at a time: per tile one
// MFMA per 16 index heads and the lane's ReLU * w partial over its four
// heads; then the sums over the four lane groups of four tiles at once with
// two lane-swap steps, which leave lane group g with the total of tile g --
// so each lane owns one score: blocks blk0 + 16 t4 + lane, stored and
// histogrammed by all 64 lanes together.
template <int kHT>
__device__ __forceinline__ void score_tiles(const KeyTiles& kt, const i32x8* qa, const int* qs,
                                            float (*wv)[4], int HT, int64_t blk0, int64_t nv,
                                            int64_t sc_ld, int lane, float* out, uint16_t* outh,
                                            int bf16, uint32_t* lh) {
  // uniform: the iteration's blocks all lie inside the (64-padded) score row,
  // so every lane stores (scores past the visible count are never read)
  const bool in_row = blk0 + kWaveTiles * 16 <= sc_ld;
  float* ob = out + blk0 + lane;
  uint16_t* obh = outh + blk0 + lane;
  const int g = lane >> 4, li = lane & 15;
#pragma unroll
  for (int t4 = 0; t4 < kWaveTiles; t4 += 4) {
    float part[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int t = t4 + u;
      // scale of (block 16t + li, group g): byte g of lane (li, u)'s dword
      // (the MFMA reads the scale operand's low byte)
      const int sc_t = __builtin_amdgcn_ds_bpermute((li + 16 * u) * 4, (int)kt.sd[t4 / 4]) >> (8 * g);
      const i32x8 kb = {(int)kt.v[t][0], (int)kt.v[t][1], (int)kt.v[t][2], (int)kt.v[t][3],
                        0, 0, 0, 0};
      float p = 0.0f;
#pragma unroll
      for (int ht = 0; ht < kHT; ht++) {
        if (ht < HT) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht], kb, acc, 4, 4, 0, qs[ht],
                                                                 0, sc_t);
          // ReLU as one integer max on the bits: a float with the sign bit
          // set is a negative integer (-0 included) and becomes +0, any
          // other is unchanged
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const float x = acc[i];       // (a vector element as an lvalue does
            const int bits = __float_as_int(x);   // not bit-cast reliably)
            p += wv[ht][i] * __builtin_bit_cast(float, bits > 0 ? bits : 0);
          }
        }
      }
      part[u] = p;
    }
    // lanes 0..31 / 32..63: tiles 0, 1 / 2, 3 summed over lane groups {0,2}, {1,3}
    const float h0 = swap_add32(part[0], part[2]);
    const float h1 = swap_add32(part[1], part[3]);
    // lane group g: tile g; block blk0 + 16 t4 + lane
    const float sc = ranked(swap_add16(h0, h1), bf16);
    const int64_t blk = blk0 + t4 * 16 + lane;
    // streaming store: the filters read each score once (and dirty L2 lines
    // would have to be written back when the kernel ends)
    if (in_row || blk < sc_ld) {
      if (bf16)
        __builtin_nontemporal_store((uint16_t)(__float_as_uint(sc) >> 16), obh + t4 * 16);
      else
        __builtin_nontemporal_store(sc, ob + t4 * 16);
    }
    // counted only when visible (an invisible block adds 0)
    atomicAdd(&lh[score_key(sc) >> kSh1], blk < nv ? 1u : 0u);
  }
}

// Workgroup w of a query covers blocks [w * iters * kIterBlocks, (w + 1) * iters * kIterBlocks).
// kParts (16 index heads, hp_ld > 0): the workgroup quantises its query heads
// itself, zeroes the query's filter counters and writes a partial histogram,
// so no kernel runs before it; otherwise the prep kernel has quantised the
// query and zeroed the global histogram the workgroup adds to.
// kIters > 0: every workgroup's range is kIters iterations (score_iters ==
// kIters) and all of them are loaded up front; 0: any count, two iterations
// in flight.
template <bool kParts, int kIters>
__global__ void __launch_bounds__(64 * kScanWaves) k_score_mx(IndexArgs a) {
  __shared__ uint32_t lh[kBins1];
  const int row = blockIdx.y;
  const int b = row / a.Q;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int64_t wg0 = (int64_t)blockIdx.x * a.score_iters * kIterBlocks;
  const size_t kb = a.pg.tab ? 0 : (size_t)b * a.cap;   // paged: rows are pool rows
  const uint8_t* kc = (const uint8_t*)a.codes + kb * 64;
  const uint8_t* ks = a.kscales + kb * 4;
  const int64_t wblk = wg0 + wave * (kWaveTiles * 16);
  // the query's operands first: loads return in order, so the query must not
  // queue behind keys
  const int64_t p_row = a.pos[row];
  constexpr int kHT = kParts ? 1 : 4;
  const int HT = kParts ? 1 : a.H / 16;
  i32x8 qa[kHT];
  int qs[kHT];
  float wv[kHT][4];
  QRaw qraw;
  if (kParts) load_q_frag(a, row, li, g, qraw);
#pragma unroll
  for (int ht = 0; ht < kHT; ht++) {
    qa[ht] = (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
    qs[ht] = 127;
#pragma unroll
    for (int i = 0; i < 4; i++) wv[ht][i] = 0.0f;
    if (ht < HT) {
      if (!kParts) {
        const uint8_t* qp = a.qmx + ((size_t)row * a.H + ht * 16 + li) * 64 + g * 16;
        u32x4 v = *(const u32x4*)qp;
        qa[ht] = (i32x8){(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        qs[ht] = a.qsc[((size_t)row * a.H + ht * 16 + li) * 4 + g];
      }
      const f32x4 w4 = *(const f32x4*)(a.w + (size_t)row * a.H + ht * 16 + g * 4);
#pragma unroll
      for (int i = 0; i < 4; i++) wv[ht][i] = w4[i];
    }
  }
  constexpr int kSets = kIters > 0 ? kIters : 2;
  KeyTiles kt[kSets];
  // paged keys, fixed iteration count: every iteration's pool row looked up
  // now, with the query loads (not one lookup wait per iteration)
  int64_t prow[kSets];
#pragma unroll
  for (int j = 0; j < kSets; j++)
    prow[j] = (kIters > 0 && a.pg.tab) ? paged_run(a.pg, b, wblk + (int64_t)j * kIterBlocks, a.cap)
                                       : -1;
  // kIters > 0: iterations 0 .. kDepth-2 go out now, iteration j + kDepth - 1
  // just before iteration j is scored (a wave that issued all its loads at
  // once would wait at the issue of the later ones -- the compute unit's
  // load queue fills -- instead of scoring what has arrived)
  constexpr int kDepth = 2;
#pragma unroll
  for (int j = 0; j < kSets; j++)
    if (kIters > 0 ? j < kDepth - 1 : j < a.score_iters)
      load_keys(kc, ks, wblk + (int64_t)j * kIterBlocks, a.cap, a.pg, b, g, li, kt[j], prow[j]);
  // the query loads went out first, so this waits for them alone and runs
  // while the first keys are on their way
  if (kParts) quantize_q_frag(a, qraw, &qa[0], &qs[0]);
  if (kParts) {
    // the filter kernels' counters of this query (they run after this kernel)
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < kBins2 + kCtr; i += gridDim.x * blockDim.x) {
      if (i < kBins2)
        a.hist2[(size_t)row * kBins2 + i] = 0u;
      else
        a.ctr[(size_t)row * kCtr + i - kBins2] = 0u;
    }
  }
  for (int i = threadIdx.x; i < kBins1; i += blockDim.x) lh[i] = 0u;
  const int64_t nv = n_visible(p_row, a.m, a.cap);
  int iters = wg0 < nv ? (int)((nv - wg0 + kIterBlocks - 1) / kIterBlocks) : 0;
  if (iters > a.score_iters) iters = a.score_iters;
  iters = __builtin_amdgcn_readfirstlane(iters);
  __syncthreads();                         // lh zeroed
  float* out = a.scores + (size_t)row * a.sc_ld;
  uint16_t* outh = (uint16_t*)a.scores + (size_t)row * a.sc_ld;
  const int bf16 = a.score_bf16;
  if (kIters > 0) {
    // every iteration's keys in flight from the start; scored in order
#pragma unroll
    for (int j = 0; j < kSets; j++) {
      if (j + kDepth - 1 < kSets)
        load_keys(kc, ks, wblk + (int64_t)(j + kDepth - 1) * kIterBlocks, a.cap, a.pg, b, g, li,
                  kt[j + kDepth - 1], prow[j + kDepth - 1]);
      if (j < iters)
        score_tiles<kHT>(kt[j], qa, qs, wv, HT, wblk + (int64_t)j * kIterBlocks, nv, a.sc_ld, lane,
                         out, outh, bf16, lh);
    }
  } else {
    // two iterations' keys in flight: kt[0] holds even, kt[1] odd iterations
    for (int it = 0; it < iters; it += 2) {
      const int64_t b0 = wblk + (int64_t)it * kIterBlocks;
      score_tiles<kHT>(kt[0], qa, qs, wv, HT, b0, nv, a.sc_ld, lane, out, outh, bf16, lh);
      if (it + 1 >= iters) break;
      if (it + 2 < iters) load_keys(kc, ks, b0 + 2 * kIterBlocks, a.cap, a.pg, b, g, li, kt[0]);
      score_tiles<kHT>(kt[1], qa, qs, wv, HT, b0 + kIterBlocks, nv, a.sc_ld, lane, out, outh, bf16,
                       lh);
      if (it + 3 < iters) load_keys(kc, ks, b0 + 3 * kIterBlocks, a.cap, a.pg, b, g, li, kt[1]);
    }
  }
  if (kParts) {
    // this workgroup's counts: row blockIdx.x of [query][workgroup][bin]
    __syncthreads();
    for (int i = threadIdx.x; i < kBins1; i += blockDim.x)
      a.hparts[((size_t)row * a.hp_ld + blockIdx.x) * kBins1 + i] = (uint16_t)lh[i];
  } else {
    hist_flush(lh, a.hist + (size_t)row * kBins1, kBins1);
  }
}

// ---------------------------------------------------------------- FP4 scan, query-tiled
// Many queries per sequence (prefill chunks): a workgroup takes kQT queries
// of one sequence and a range of kQRange blocks, so every key fragment loaded
// feeds kQT MFMAs (one per query).  Wave w takes the 16-block tiles w, w+4,
// ... of the range; per tile and query one v_mfma_scale_f32_16x16x128_f8f6f4
// (M = the 16 index heads, N = 16 blocks), ReLU * w over each lane's four
// heads, then the sum over the four lane groups for all kQT queries at once
// with two lane-swap steps (v_permlane32_swap, v_permlane16_swap), which
// leaves lane group g with the totals of queries (g & 1) + 4 (g >> 1) and
// that + 2.  Per-query first-digit histograms in LDS, flushed once.
constexpr int kQRange = 16384;

struct QFrag {
  u32x4 v;
  int sc;
};

__device__ __forceinline__ void load_qfrag(const uint8_t* kc, const uint8_t* ks, int64_t blk,
                                           int64_t last, int g, QFrag& f, const int* pgl,
                                           int64_t r0, int psh) {
  int64_t bb = blk < last ? blk : last;     // clamped: always a real row
  if (pgl) bb = ((int64_t)pgl[(bb - r0) >> psh] << psh) | (bb & (((int64_t)1 << psh) - 1));
  // a plain load: every query tile of the sequence reads these keys again
  f.v = *(const u32x4*)(kc + bb * 64 + g * 16);
  f.sc = ks[bb * 4 + g];
}

// kMode: kModeStore writes every score and the first-digit histogram (the
// full-score path; with fb_only only for workgroups holding a row that the
// sampled selection handed over); kModeSample scores the sample tiles into
// the sample rows; kModeCollect scores every block and appends those at or
// above the row's sampled threshold to its candidate list.
constexpr int kModeStore = 0, kModeSample = 1, kModeCollect = 2;
// Word 3 of a raw (untyped, byte-addressed) buffer resource on this
// architecture: 32-bit data format, no swizzle, no index stride.
constexpr int kBufDword3 = 0x00020000;

// A pointer whose value is the same in every lane, held in scalar registers.
__device__ __forceinline__ void* wg_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void*)(((uint64_t)hi << 32) | lo);
}
constexpr int kCollectPer = 6;             // LDS candidate slots per lane and query

__device__ __forceinline__ void load_qfrag_s(const IndexArgs& a, const uint8_t* kc, const uint8_t* ks,
                                             int b, int64_t sb, int64_t last, int g, QFrag& f) {
  const int64_t s = sb < last ? sb : last;  // clamped: always a real sample block
  int64_t bb = ((s >> 4) << 8) | (s & 15);
  if (a.pg.tab) bb = page_row(a.pg, b, bb);
  f.v = *(const u32x4*)(kc + bb * 64 + g * 16);
  f.sc = ks[bb * 4 + g];
}

// One query's 16-head x 16-block MXFP4 product; the query scale is byte
// `sel` of the register sa (four queries' scales share a register).
template <int kSel>
__device__ __forceinline__ f32x4 mfma_q_sel(const i32x8& a, const i32x8& b, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, (f32x4){0.f, 0.f, 0.f, 0.f}, 4, 4,
                                                          kSel, sa, 0, sb);
}
__device__ __forceinline__ f32x4 mfma_q_scaled(int sel, const i32x8& a, const i32x8& b, int sa, int sb) {
  switch (sel) {
    case 0: return mfma_q_sel<0>(a, b, sa, sb);
    case 1: return mfma_q_sel<1>(a, b, sa, sb);
    case 2: return mfma_q_sel<2>(a, b, sa, sb);
    default: return mfma_q_sel<3>(a, b, sa, sb);
  }
}

template <int kMode, bool kBf16>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
k_score_mx_q(IndexArgs a) {
  __shared__ uint32_t lh[kQT][kBins1];
  __shared__ int pg_rows[kQRange / 128];    // paged keys: the range's pool pages
  // collect: each lane's candidates of its two queries in slots of its own
  // (counted in registers: no atomic in the scoring loop), gathered per
  // query at the end with one global reservation.  A slot holds the raw
  // pair (score bits, block offset within the range); the 64-bit selection
  // key is built when the slots are gathered, off the scoring loop.
  __shared__ uint64_t cbuf[kMode == kModeCollect ? 256 * 2 * kCollectPer : 1];
  __shared__ uint32_t lcnt[kMode == kModeCollect ? 512 : 1], loff[kMode == kModeCollect ? 512 : 1];
  __shared__ uint32_t cbase[kQT];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int qtiles = (a.Q + kQT - 1) / kQT;
  const int b = blockIdx.x / qtiles;
  const int t0 = (blockIdx.x % qtiles) * kQT;
  const int64_t r0 = (int64_t)blockIdx.y * kQRange;
  int64_t nv_max = 0;
  bool any_fb = false;
#pragma unroll
  for (int q = 0; q < kQT; q++) {
    const int t = t0 + q;
    int64_t nv = t < a.Q ? n_visible(a.pos[(int64_t)b * a.Q + t], a.m, a.cap) : 0;
    if (kMode == kModeSample) nv = n_sampled(nv);
    nv_max = nv > nv_max ? nv : nv_max;
    if (kMode == kModeStore && a.fb_only && t < a.Q)
      any_fb = any_fb || a.ctr[((int64_t)b * a.Q + t) * kCtr + kFbSlot] != 0u;
  }
  if (kMode == kModeStore && a.fb_only && !any_fb) return;   // uniform
  if (r0 >= nv_max) return;                // uniform across the workgroup
  for (int i = threadIdx.x; i < kQT * kBins1; i += blockDim.x) (&lh[0][0])[i] = 0u;
  if (a.pg.tab && kMode != kModeSample) {
    // (a page longer than the range: the range lies in one page)
    const int n_pg = (kQRange >> a.pg.psh) > 0 ? (kQRange >> a.pg.psh) : 1;
    for (int i = threadIdx.x; i < n_pg; i += blockDim.x) {
      int64_t lp = (r0 >> a.pg.psh) + i;
      lp = lp < a.pg.tab_ld ? lp : a.pg.tab_ld - 1;
      int64_t pp = a.pg.tab[(int64_t)b * a.pg.tab_ld + lp];
      pp = pp < 0 ? 0 : (pp >= a.pg.n_pages ? a.pg.n_pages - 1 : pp);
      pg_rows[i] = (int)pp;
    }
  }
  // A operands (16 heads x 128 elements of each query), scales, head weights
  i32x8 qa[kQT];
  int qs[kQT / 4];                         // the queries' scale bytes, four per register
  // head weights in LDS (read per tile, four heads of one query per lane:
  // the lanes of a group read one address), not in 32 registers
  __shared__ float lw[kQT][16];
  if (threadIdx.x < kQT * 16) {
    const int q = threadIdx.x >> 4, h = threadIdx.x & 15, t = t0 + q;
    lw[q][h] = t < a.Q ? a.w[((int64_t)b * a.Q + t) * 16 + h] : 0.0f;
  }
#pragma unroll
  for (int q = 0; q < kQT; q++) {
    const int t = t0 + q;
    const int64_t row = (int64_t)b * a.Q + (t < a.Q ? t : a.Q - 1);
    u32x4 v = *(const u32x4*)(a.qmx + (row * 16 + li) * 64 + g * 16);
    qa[q] = (i32x8){(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
    const int sb = a.qsc[(row * 16 + li) * 4 + g];
    if (q % 4 == 0) qs[q / 4] = sb;
    else qs[q / 4] |= sb << (8 * (q % 4));
  }
  // the two queries this lane stores: (g & 1) + 4 (g >> 1) and that + 2
  const int qa0 = (g & 1) + 4 * (g >> 1), qa1 = qa0 + 2;
  int64_t nv0 = 0, nv1 = 0;
#pragma unroll
  for (int q = 0; q < kQT; q++) {
    const int t = t0 + q;
    int64_t nv = t < a.Q ? n_visible(a.pos[(int64_t)b * a.Q + t], a.m, a.cap) : 0;
    if (kMode == kModeSample) nv = n_sampled(nv);
    if (q == qa0) nv0 = nv;
    if (q == qa1) nv1 = nv;
  }
  // collect: the two rows' thresholds and counters
  const int64_t row0 = (int64_t)b * a.Q + t0 + qa0, row1 = (int64_t)b * a.Q + t0 + qa1;
  uint32_t thr0 = 0xFFFFFFFFu, thr1 = 0xFFFFFFFFu;
  float thf0, thf1;                        // the thresholds as scores (one compare per score)
  if (kMode == kModeCollect) {
    if (t0 + qa0 < a.Q) thr0 = a.ctr[row0 * kCtr + kThrSlot];
    if (t0 + qa1 < a.Q) thr1 = a.ctr[row1 * kCtr + kThrSlot];
  }
  thf0 = key_floor(thr0);
  thf1 = key_floor(thr1);
  // a candidate of this lane's query `which` (0: qa0, 1: qa1): its next own
  // slot, or (its slots full) a global one
  uint32_t cn[2] = {0u, 0u};
  auto put_cand = [&](int which, int64_t row, float sc, int rel) {
    if (cn[which] < (uint32_t)kCollectPer) {
      cbuf[(threadIdx.x * 2 + which) * kCollectPer + cn[which]] =
          ((uint64_t)(uint32_t)rel << 32) | __float_as_uint(sc);
      cn[which]++;
    } else {
      const uint32_t gs = atomicAdd(&a.ctr[row * kCtr + kCntSlot], 1u);
      if (gs < (uint32_t)kCandCap) a.cand[row * kCandCap + gs] = sel_key(score_key(sc), r0 + rel);
    }
  };
  const size_t o0 = (size_t)((int64_t)b * a.Q + t0 + qa0) * a.sc_ld;   // score row offsets
  const size_t o1 = (size_t)((int64_t)b * a.Q + t0 + qa1) * a.sc_ld;
  __syncthreads();                         // lh zeroed

  const size_t kb = a.pg.tab ? 0 : (size_t)b * a.cap;   // paged: rows are pool rows
  const uint8_t* kc = (const uint8_t*)a.codes + kb * 64;
  const uint8_t* ks = a.kscales + kb * 4;
  const int* pgl = a.pg.tab ? pg_rows : nullptr;
  const int psh = a.pg.psh;
  const int64_t r1 = r0 + kQRange < nv_max ? r0 + kQRange : nv_max;
  const int64_t last = r1 - 1;
  // Blocks are counted from r0 in 32 bits inside the loop: the range's
  // length, and per stored row its visible blocks past r0 (0 for a row
  // past Q), so a bounds test is one 32-bit compare and an unpaged key
  // load one 32-bit offset from the range's base.
  const int nrel = (int)(r1 - r0), lastr = nrel - 1;
  auto rel_bound = [&](int64_t nv, bool ok) -> int {
    const int64_t v = ok ? nv - r0 : 0;
    return v <= 0 ? 0 : (v > kQRange ? kQRange : (int)v);
  };
  const int nb0 = rel_bound(nv0, t0 + qa0 < a.Q), nb1 = rel_bound(nv1, t0 + qa1 < a.Q);
  // unpaged: the range's keys and scales as two buffer resources (base in
  // scalar registers -- the values are the workgroup's, readfirstlane tells
  // the compiler so -- and the lane's 32-bit byte offset the only address
  // work; every offset used is below the range's length)
  const int nrel_s = __builtin_amdgcn_readfirstlane(nrel);
  const __amdgpu_buffer_rsrc_t kcr =
      __builtin_amdgcn_make_buffer_rsrc(wg_ptr(kc + (size_t)r0 * 64), 0, nrel_s * 64, kBufDword3);
  const __amdgpu_buffer_rsrc_t ksr =
      __builtin_amdgcn_make_buffer_rsrc(wg_ptr(ks + (size_t)r0 * 4), 0, nrel_s * 4, kBufDword3);

  auto tile = [&](const QFrag& f, int rel0) {
    const i32x8 kb = {(int)f.v[0], (int)f.v[1], (int)f.v[2], (int)f.v[3], 0, 0, 0, 0};
    // the eight queries' products first, each into its own accumulator, so
    // that the MFMAs issue back to back and the epilogue reads finished ones
    // in two batches of four queries (register room for four waves per SIMD)
    float part[kQT];
#pragma unroll
    for (int hq = 0; hq < kQT; hq += 4) {
    f32x4 acc[kQT];
    // (the batch's MFMAs issue at raised wave priority, ahead of the other
    // waves' VALU epilogues: collect scan 1.77 -> 1.74-1.78 ms, a gain within
    // the spread between runs)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int q = hq; q < hq + 4; q++)
      acc[q] = mfma_q_scaled(q % 4, qa[q], kb, qs[q / 4], f.sc);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int q = hq; q < hq + 4; q++) {
      // ReLU as one integer max on the bits (a float with the sign bit set
      // is a negative integer and becomes +0); w-weighted sum of the lane's
      // four heads
      float r[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float x = acc[q][i];
        const int bits = __float_as_int(x);
        r[i] = __int_as_float(bits > 0 ? bits : 0);
      }
      const f32x4 wq = *(const f32x4*)&lw[q][g * 4];
      float p = wq[0] * r[0];
#pragma unroll
      for (int i = 1; i < 4; i++) p = fmaf(wq[i], r[i], p);
      part[q] = p;
    }
    }
    // sum over the four lane groups, all queries at once
    float h[4];
#pragma unroll
    for (int j = 0; j < 4; j++) h[j] = swap_add32(part[j], part[4 + j]);
    const float s0 = ranked(swap_add16(h[0], h[1]), kBf16);   // queries 0, 1, 4, 5 by lane group
    const float s1 = ranked(swap_add16(h[2], h[3]), kBf16);   // queries 2, 3, 6, 7
    const int rel = rel0 + li;
    const int64_t blk = r0 + rel;
    if (kMode == kModeStore) {
      if (rel < nb0) {
        put_score(a, o0 + blk, s0);
        atomicAdd(&lh[qa0][score_key(s0) >> kSh1], 1u);
      }
      if (rel < nb1) {
        put_score(a, o1 + blk, s1);
        atomicAdd(&lh[qa1][score_key(s1) >> kSh1], 1u);
      }
    } else if (kMode == kModeSample) {
      if (rel < nb0) a.samp[row0 * a.samp_ld + blk] = s0;
      if (rel < nb1) a.samp[row1 * a.samp_ld + blk] = s1;
    } else {
      // (few pass: about 1.3 % of the scores at the benchmark's shape)
      if (rel < nb0 && s0 >= thf0) put_cand(0, row0, s0, rel);
      if (rel < nb1 && s1 >= thf1) put_cand(1, row1, s1, rel);
    }
  };

  // tiles w, w + 4, ... of 16 blocks; two fragments in flight
  auto ld = [&](int rel, QFrag& f) {
    if (kMode == kModeSample) {
      load_qfrag_s(a, kc, ks, b, r0 + rel, last, g, f);
    } else if (pgl) {
      load_qfrag(kc, ks, r0 + rel, last, g, f, pgl, r0, psh);
    } else {
      // clamped: always a real row; a plain load (every query tile of the
      // sequence reads these keys again)
      const int o = rel < lastr ? rel : lastr;
      f.v = __builtin_amdgcn_raw_buffer_load_b128(kcr, o * 64 + g * 16, 0, 0);
      f.sc = __builtin_amdgcn_raw_buffer_load_b8(ksr, o * 4 + g, 0, 0);
    }
  };
  QFrag fa, fb;
  int rel0 = wave * 16;
  ld(rel0 + li, fa);
  for (; rel0 < nrel; rel0 += 128) {
    ld(rel0 + 64 + li, fb);
    tile(fa, rel0);
    if (rel0 + 64 >= nrel) break;
    ld(rel0 + 128 + li, fa);
    tile(fb, rel0 + 64);
  }
  if (kMode == kModeCollect) {
    const int t = threadIdx.x;
    lcnt[2 * t] = cn[0] < (uint32_t)kCollectPer ? cn[0] : (uint32_t)kCollectPer;
    lcnt[2 * t + 1] = cn[1] < (uint32_t)kCollectPer ? cn[1] : (uint32_t)kCollectPer;
    __syncthreads();
    if (t < kQT) {
      // query q is held by lane group g of every wave as its query `which`
      const int q = t, which = (q >> 1) & 1, qb = q - 2 * which;
      const int gq = (qb & 1) + 2 * (qb >> 2);
      uint32_t tot = 0;
      for (int w = 0; w < 4; w++)
        for (int l = 0; l < 16; l++) {
          const int idx = 2 * (w * 64 + gq * 16 + l) + which;
          loff[idx] = tot;
          tot += lcnt[idx];
        }
      cbase[q] = (tot && t0 + q < a.Q) ? atomicAdd(&a.ctr[((int64_t)b * a.Q + t0 + q) * kCtr + kCntSlot], tot)
                                       : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int which = 0; which < 2; which++) {
      const int q = which ? qa1 : qa0;
      if (t0 + q >= a.Q) continue;
      const int idx = 2 * t + which;
      const uint32_t base = cbase[q] + loff[idx];
      uint64_t* dst = a.cand + ((int64_t)b * a.Q + t0 + q) * kCandCap;
      for (uint32_t j = 0; j < lcnt[idx]; j++)
        if (base + j < (uint32_t)kCandCap) {
          const uint64_t raw = cbuf[idx * kCollectPer + j];
          dst[base + j] = sel_key(score_key(__uint_as_float((uint32_t)raw)), r0 + (int64_t)(raw >> 32));
        }
    }
  }
  if (kMode != kModeStore) return;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kQT; q++) {
    if (t0 + q >= a.Q) break;
    uint32_t* gh = a.hist + ((int64_t)b * a.Q + t0 + q) * kBins1;
    for (int i = threadIdx.x; i < kBins1; i += blockDim.x) {
      const uint32_t c = lh[q][i];
      if (c) atomicAdd(gh + i, c);
    }
  }
}

// ---------------------------------------------------------------- fp32 scan
__global__ void __launch_bounds__(256) k_score_f32(IndexArgs a) {
  extern __shared__ float qsm[];          // [H][d], w[H], then the histogram
  const int row = blockIdx.y;
  const int b = row / a.Q;
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int64_t wg0 = (int64_t)blockIdx.x * blockDim.x;
  if (wg0 >= nv) return;
  const int64_t blk = wg0 + threadIdx.x;
  float* wsm = qsm + a.H * a.d;
  uint32_t* lh = (uint32_t*)(wsm + a.H);
  for (int i = threadIdx.x; i < kBins1; i += blockDim.x) lh[i] = 0u;
  for (int i = threadIdx.x; i < a.H * a.d; i += blockDim.x)
    qsm[i] = load_as_f32(a.q, a.q_bf16, (size_t)row * a.H * a.d + i);
  for (int i = threadIdx.x; i < a.H; i += blockDim.x) wsm[i] = a.w[(size_t)row * a.H + i];
  __syncthreads();
  if (blk < nv) {
    const float* kr = (const float*)a.codes + ((size_t)b * a.cap + blk) * a.d;
    float s = 0.0f;
    for (int h = 0; h < a.H; h++) {
      float dot = 0.0f;
      for (int c = 0; c < a.d; c++) dot += qsm[h * a.d + c] * kr[c];
      s += wsm[h] * fmaxf(dot, 0.0f);
    }
    const float r = ranked(s, a.score_bf16);
    put_score(a, (size_t)row * a.sc_ld + blk, r);
    atomicAdd(&lh[score_key(r) >> kSh1], 1u);
  }
  hist_flush(lh, a.hist + (size_t)row * kBins1, kBins1);
}

// ---------------------------------------------------------------- filter + select

// This thread's kPer consecutive scores of filter chunk `chunk`, in two
// halves so that the loads can be issued before anything else the kernel
// waits for: issue_group needs no visible count (the score rows are padded to
// 64 entries; a group past the padded row reads the row's first group),
// finish_group converts them to keys and returns how many are below nv.
// kBf16: the rows hold bf16 scores (32 bytes per group instead of 64).
struct Group {
  u32x4 v[kPer / 4];
  int64_t g0;
};

template <bool kBf16>
__device__ __forceinline__ void issue_group(const IndexArgs& a, int row, int chunk, Group& gr) {
  gr.g0 = (int64_t)chunk * kFilterChunk + threadIdx.x * kPer;
  const size_t off = (size_t)row * a.sc_ld + (gr.g0 < a.sc_ld ? gr.g0 : 0);
  if (kBf16) {
    const uint16_t* sc = (const uint16_t*)a.scores + off;
#pragma unroll
    for (int j = 0; j < kPer / 8; j++) gr.v[j] = *(const u32x4*)(sc + 8 * j);
  } else {
    const float* sc = a.scores + off;
#pragma unroll
    for (int j = 0; j < kPer / 4; j++) gr.v[j] = *(const u32x4*)(sc + 4 * j);
  }
}

template <bool kBf16>
__device__ __forceinline__ int finish_group(const Group& gr, int64_t nv, uint32_t* k32) {
  const int64_t rem = nv - gr.g0;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    float f;
    if (kBf16) {
      const uint32_t w = gr.v[j / 8][(j % 8) / 2];
      f = bf16_to_f32((j & 1) ? (w >> 16) : (w & 0xFFFFu));
    } else {
      const uint32_t w = gr.v[j / 4][j % 4];
      f = __uint_as_float(w);
    }
    k32[j] = score_key(f);
  }
  return rem <= 0 ? 0 : (rem >= kPer ? kPer : (int)rem);
}

// Common head of the filter kernels: the query's visible count, its k', and
// the first-digit threshold bin from the score histogram.
struct FilterRow {
  int64_t nv;
  int kk;
  uint32_t b1, above1;
};

__device__ __forceinline__ bool filter_head(const IndexArgs& a, int row, uint32_t* lh,
                                            uint32_t* tmp, FilterRow* fr) {
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  fr->nv = n_visible(a.pos[row], a.m, a.cap);
  fr->kk = (int)(fr->nv < a.k ? fr->nv : a.k);
  if (fr->kk == fr->nv) return false;
  if ((int64_t)blockIdx.x * kFilterChunk >= fr->nv) return false;
  const uint32_t* gh = a.hist + (size_t)row * kBins1;
  for (int i = threadIdx.x; i < kBins1; i += blockDim.x) lh[i] = gh[i];
  __syncthreads();
  find_bin(lh, kBins1, (uint32_t)fr->kk, tmp, &s_bin, &s_above);
  fr->b1 = (uint32_t)s_bin;
  fr->above1 = s_above;
  return true;
}

// Partial first-digit histograms of a query: one row of 256 16-bit counts
// per scan workgroup ([query][workgroup][bin], at most kMaxParts rows).  A
// load step reads 8 rows with the 256 threads in contiguous 16-byte pieces:
// thread t takes bins 8 (t % 32) .. +7 of row 8i + t / 32 in step i, so a
// thread always sums the same 8 bins.
struct Parts {
  u32x4 v[kMaxParts / 8];
};

__device__ __forceinline__ void load_parts(const IndexArgs& a, int row, Parts& p) {
  const int t = threadIdx.x;
  const uint16_t* base = a.hparts + (size_t)row * a.hp_ld * kBins1 + 8 * (t % 32);
#pragma unroll
  for (int i = 0; i < kMaxParts / 8; i++) {
    const int slot = 8 * i + t / 32;
    p.v[i] = slot < a.score_wgs ? *(const u32x4*)(base + (size_t)slot * kBins1)
                                : (u32x4){0u, 0u, 0u, 0u};
  }
}

// The count of bin threadIdx.x over all rows; red = 8 x 256 words of LDS
// (free again on return).
__device__ __forceinline__ uint32_t part_sum(const Parts& p, uint32_t* red) {
  const int t = threadIdx.x;
  uint32_t acc[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kMaxParts / 8; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      acc[2 * j] += p.v[i][j] & 0xFFFFu;
      acc[2 * j + 1] += p.v[i][j] >> 16;
    }
#pragma unroll
  for (int j = 0; j < 8; j++) red[(t / 32) * kBins1 + 8 * (t % 32) + j] = acc[j];
  __syncthreads();
  uint32_t sum = 0;
#pragma unroll
  for (int k = 0; k < 8; k++) sum += red[k * kBins1 + t];
  __syncthreads();
  return sum;
}

template <bool kBf16>
__device__ __forceinline__ void filter1_row(const IndexArgs& a, const int row) {
  __shared__ uint32_t lh[kBins2];
  __shared__ uint32_t tmp[kFThreads / 64];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  // all global loads first, before the query position arrives (no address
  // depends on it): the first histogram (bin = thread), this thread's scores
  Parts pt;
  uint32_t h1 = 0;
  Group gr;
  if (a.hp_ld)
    load_parts(a, row, pt);
  else
    h1 = a.hist[(size_t)row * kBins1 + threadIdx.x];   // kBins1 == kFThreads
  issue_group<kBf16>(a, row, blockIdx.x, gr);
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int kk = (int)(nv < a.k ? nv : a.k);
  if (kk == nv) {                          // everything visible is selected
    if (blockIdx.x == 0) {
      int32_t* out = a.topk + (size_t)row * a.k;
      for (int64_t i = threadIdx.x; i < a.k; i += blockDim.x) out[i] = i < nv ? (int32_t)i : -1;
    }
    return;
  }
  if ((int64_t)blockIdx.x * kFilterChunk >= nv) return;
  static_assert(8 * kBins1 <= kBins2, "partial-sum scratch fits the histogram buffer");
  if (a.hp_ld) h1 = part_sum(pt, lh);
  lh[threadIdx.x] = h1;
  __syncthreads();
  find_bin(lh, kBins1, (uint32_t)kk, tmp, &s_bin, &s_above);
  const uint32_t b1 = (uint32_t)s_bin;
  // the first digit for the kernels that follow
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.ctr[(size_t)row * kCtr + 4] = b1;
    a.ctr[(size_t)row * kCtr + 5] = s_above;
  }
  for (int i = threadIdx.x; i < kBins2; i += blockDim.x) lh[i] = 0u;
  uint32_t k32[kPer];
  const int n_in = finish_group<kBf16>(gr, nv, k32);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; j++)
    if (j < n_in && (k32[j] >> kSh1) == b1) atomicAdd(&lh[(k32[j] >> kSh2) & (kBins2 - 1)], 1u);
  hist_flush(lh, a.hist2 + (size_t)row * kBins2, kBins2);
}

template <bool kBf16>
__global__ void __launch_bounds__(kFThreads) k_filter1(IndexArgs a) {
  if (!a.fb_only) {
    filter1_row<kBf16>(a, (int)blockIdx.y);
    return;
  }
  // the rows the sampled selection handed over, gridDim.y at a time
  const uint32_t n_fb = a.fbl[0];
  for (uint32_t r = blockIdx.y; r < n_fb; r += gridDim.y) {
    filter1_row<kBf16>(a, (int)a.fbl[1 + r]);
    __syncthreads();
  }
}

// Candidate appends go to an LDS buffer first (wave-aggregated LDS atomics);
// the workgroup then reserves its range in the query's global list with a
// single atomic.  Lanes that find the LDS buffer full append to the global
// list directly.
constexpr int kCandLds = 1024;

struct CandList {
  uint64_t* buf;
  uint32_t* count;                         // LDS counter

  __device__ __forceinline__ void append(bool flag, uint64_t value, uint32_t* gcount,
                                         uint64_t* gbuf) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint64_t mask = __builtin_amdgcn_ballot_w64(flag);
    if (!mask) return;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(count, (uint32_t)__builtin_popcountll(mask));
    base = __shfl(base, 0, 64);
    uint32_t slot = base + (uint32_t)__builtin_popcountll(mask & below);
    bool spill = flag && slot >= (uint32_t)kCandLds;
    if (flag && !spill) buf[slot] = value;
    uint64_t ms = __builtin_amdgcn_ballot_w64(spill);
    if (!ms) return;
    uint32_t gb = 0;
    if (lane == 0) gb = atomicAdd(gcount, (uint32_t)__builtin_popcountll(ms));
    gb = __shfl(gb, 0, 64);
    if (spill) {
      uint32_t gs = gb + (uint32_t)__builtin_popcountll(ms & below);
      if (gs < (uint32_t)kCandCap) gbuf[gs] = value;
    }
  }

  // all threads; copies the buffered entries to the global list
  __device__ __forceinline__ void flush(uint32_t* gcount, uint64_t* gbuf, uint32_t* s_base) {
    __syncthreads();
    uint32_t n = *count < (uint32_t)kCandLds ? *count : (uint32_t)kCandLds;
    if (threadIdx.x == 0) *s_base = n ? atomicAdd(gcount, n) : 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x)
      if (*s_base + i < (uint32_t)kCandCap) gbuf[*s_base + i] = buf[i];
  }
};

__device__ __forceinline__ void filter2_row(const IndexArgs& a, const int row) {
  __shared__ uint32_t lh[kBins2];
  __shared__ uint32_t tmp[kFThreads / 64];
  __shared__ uint64_t cand_buf[kCandLds];
  __shared__ int s_bin;
  __shared__ uint32_t s_above, cand_n, s_base;
  // all global loads first, before the query position arrives: the first
  // digit (published by k_filter1), the second histogram, this thread's scores
  uint32_t* ctr = a.ctr + (size_t)row * kCtr;
  const uint32_t b1 = ctr[4], above1 = ctr[5];
  constexpr int kPer2 = kBins2 / kFThreads;                          // 8
  const u32x4* gh2 = (const u32x4*)(a.hist2 + (size_t)row * kBins2 + threadIdx.x * kPer2);
  const u32x4 h2a = gh2[0], h2b = gh2[1];
  Group gr;
  issue_group<false>(a, row, blockIdx.x, gr);
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int kk = (int)(nv < a.k ? nv : a.k);
  if (kk == nv || (int64_t)blockIdx.x * kFilterChunk >= nv) return;
  if (threadIdx.x == 0) cand_n = 0;
  *(u32x4*)&lh[threadIdx.x * kPer2] = h2a;
  *(u32x4*)&lh[threadIdx.x * kPer2 + 4] = h2b;
  __syncthreads();
  find_bin(lh, kBins2, (uint32_t)kk - above1, tmp, &s_bin, &s_above);
  const uint32_t b12 = (b1 << 11) | (uint32_t)s_bin;   // key bits 31..13
  uint32_t k32[kPer];
  const int n_in = finish_group<false>(gr, nv, k32);
  const int64_t i0 = gr.g0;
  FilterRow fr{nv, kk, b1, above1};
  uint64_t* cand = a.cand + (size_t)row * kCandCap;
  CandList cnd{cand_buf, &cand_n};
  uint32_t above = 0;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const bool in = j < n_in;
    const uint32_t d12 = k32[j] >> kSh2;
    above += (in && d12 > b12) ? 1u : 0u;
    cnd.append(in && d12 == b12, sel_key(k32[j], i0 + j), ctr + 0, cand);
  }
  cnd.flush(ctr + 0, cand, &s_base);
  if (a.elist) {
    // fused with the CSA attention: the chunk's selection keys of every id
    // at or above the candidates' bin (the ids above it and the
    // candidates), in id order; the attention filters them by the exact
    // threshold in place of the emit step.  One scan gives both the list
    // positions (low half) and the count above the bin (high half); both
    // stay below 2^16 (4096 ids a chunk).
    uint32_t ecnt = 0;
#pragma unroll
    for (int j = 0; j < kPer; j++) ecnt += (j < n_in && (k32[j] >> kSh2) >= b12) ? 1u : 0u;
    const uint32_t packed = (above << 16) | ecnt;
    uint32_t tot;
    uint32_t epos = (block_incl_scan(packed, tmp, &tot) - packed) & 0xFFFFu;
    const size_t ci = (size_t)row * n_chunks(a.cap) + blockIdx.x;
    uint64_t* el = a.elist + ci * kFilterChunk;
#pragma unroll
    for (int j = 0; j < kPer; j++)
      if (j < n_in && (k32[j] >> kSh2) >= b12) el[epos++] = sel_key(k32[j], i0 + j);
    if (threadIdx.x == 0) a.elen[ci] = tot & 0xFFFFu;
    above = tot >> 16;
  } else {
    // the chunk's count of ids above the candidates' bin
    above = block_sum(above, tmp);
  }
  // the threshold digits
  if (threadIdx.x == 0) {
    a.chunk[(size_t)row * n_chunks(a.cap) + blockIdx.x] = above;
    if (blockIdx.x == 0) {
      ctr[2] = b12;
      ctr[3] = (uint32_t)fr.kk - fr.above1 - s_above;   // candidates to take
    }
  }
}

__global__ void __launch_bounds__(kFThreads) k_filter2(IndexArgs a) {
  if (!a.fb_only) {
    filter2_row(a, (int)blockIdx.y);
    return;
  }
  // the rows the sampled selection handed over, gridDim.y at a time
  const uint32_t n_fb = a.fbl[0];
  for (uint32_t r = blockIdx.y; r < n_fb; r += gridDim.y) {
    filter2_row(a, (int)a.fbl[1 + r]);
    __syncthreads();
  }
}

// Every workgroup of a query resolves the threshold T from the candidates
// (few: they share the top 19 key bits with the k-th largest score), finds
// its chunk's output offset, and writes its chunk's selected ids in order.
__device__ __forceinline__ void emit_row(const IndexArgs& a, const int row) {
  __shared__ uint32_t lh[kBinsMax];
  __shared__ uint32_t tmp[kFThreads / 64];
  __shared__ uint64_t cl[kEmitCand];
  // all global loads first, before the query position arrives: counters, the
  // first candidates (speculatively: the list always has kCandCap slots), the
  // earlier chunks' counts, scores
  const uint32_t* ctr = a.ctr + (size_t)row * kCtr;
  const uint32_t n_cand = ctr[0], b12 = ctr[2], need = ctr[3];
  const uint64_t* gc = a.cand + (size_t)row * kCandCap;
  const uint64_t c_first = gc[threadIdx.x];
  const uint32_t* cc = a.chunk + (size_t)row * n_chunks(a.cap);
  const uint32_t cc_first = (int)threadIdx.x < (int)blockIdx.x ? cc[threadIdx.x] : 0u;
  Group gr;
  issue_group<false>(a, row, blockIdx.x, gr);
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int kk = (int)(nv < a.k ? nv : a.k);
  if (kk == nv) return;                    // written by k_filter1
  int32_t* out = a.topk + (size_t)row * a.k;
  if (blockIdx.x == 0)
    for (int i = kk + threadIdx.x; i < a.k; i += blockDim.x) out[i] = -1;
  if ((int64_t)blockIdx.x * kFilterChunk >= nv) return;
  const bool in_lds = n_cand <= (uint32_t)kEmitCand;
  if (in_lds) {
    if (threadIdx.x < n_cand) cl[threadIdx.x] = c_first;
    for (uint32_t i = threadIdx.x + blockDim.x; i < n_cand; i += blockDim.x) cl[i] = gc[i];
  }
  __syncthreads();
  const CandSrc src{in_lds ? cl : nullptr, gc, n_cand, a.scores + (size_t)row * a.sc_ld, nv, b12,
                    32 - kSh2, n_cand <= (uint32_t)kCandCap};
  const uint64_t T = (src.compact && in_lds && n_cand <= (uint32_t)kRankCand)
                         ? rank_threshold(cl, n_cand, need)
                         : resolve_threshold(src, need, lh, tmp);
  // offset of this chunk: ids above the bin in earlier chunks, plus the
  // candidates >= T with lower ids
  const int64_t c0 = (int64_t)blockIdx.x * kFilterChunk;
  uint32_t before = cc_first;
  for (int c = threadIdx.x + blockDim.x; c < (int)blockIdx.x; c += blockDim.x) before += cc[c];
  const int64_t n = src.size();
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    uint64_t key;
    if (src.get(i, &key) && key >= T) {
      const int64_t id = (int64_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
      before += id < c0 ? 1u : 0u;
    }
  }
  uint32_t k32[kPer];
  const int n_in = finish_group<false>(gr, nv, k32);
  const int64_t i0 = gr.g0;
  uint32_t sel = 0;
#pragma unroll
  for (int j = 0; j < kPer; j++)
    if (j < n_in && sel_key(k32[j], i0 + j) >= T) sel |= 1u << j;
  const uint32_t cnt = (uint32_t)__builtin_popcount(sel);
  // one scan for both: the chunk's offset (sum of `before`, high half) and
  // this thread's rank in the chunk (prefix of `cnt`, low half); both sums
  // stay below 2^16 (k <= 4096)
  const uint32_t packed = (before << 16) | cnt;
  uint32_t total;
  const uint32_t incl = block_incl_scan(packed, tmp, &total);
  uint32_t pos = (total >> 16) + ((incl - packed) & 0xFFFFu);
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    if ((sel >> j) & 1u) {
      if (pos < (uint32_t)kk) out[pos] = (int32_t)(i0 + j);
      pos++;
    }
  }
}

__global__ void __launch_bounds__(kFThreads) k_emit(IndexArgs a) {
  if (!a.fb_only) {
    emit_row(a, (int)blockIdx.y);
    return;
  }
  // the rows the sampled selection handed over, gridDim.y at a time
  const uint32_t n_fb = a.fbl[0];
  for (uint32_t r = blockIdx.y; r < n_fb; r += gridDim.y) {
    emit_row(a, (int)a.fbl[1 + r]);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- sampled-threshold selection
// Query-tiled scans (prefill chunks) do not materialise the score matrix
// (4 bytes per query and block, written once and read three times by the
// filters above).  A sample pass scores every 16th tile of 16 blocks; for
// each query k_thresh takes the r-th largest sample key as a lower bound L,
// with r = k s/n + 6 sqrt(k s/n) + 16 for s samples of n visible blocks
// (about 6 standard deviations above the expected sample count of the top
// k), so that at least k of all keys are >= L with near certainty and
// about r n / s are; the collect pass scores every block and appends those
// >= L to the query's candidate list; k_select_pf takes the exact top k of
// the candidates (the same 64-bit keys and tie rule as the filters) and
// emits them in ascending id order from an id bitmap.  A query whose
// candidates are fewer than k or more than the list holds (ties, or a
// sample unlike the rest) is flagged and runs through the full-score path
// (store scan + the three filters, each skipping unflagged rows), so the
// result is exact whatever the scores.
__global__ void __launch_bounds__(kFThreads) k_thresh(IndexArgs a) {
  __shared__ uint32_t lh[kBins2];
  __shared__ uint32_t tmp[kFThreads / 64];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int kk = (int)(nv < a.k ? nv : a.k);
  uint32_t* ctr = a.ctr + (size_t)row * kCtr;
  const int64_t ns = n_sampled(nv);
  const float ksf = nv > 0 ? (float)kk * (float)ns / (float)nv : 0.0f;
  const int64_t r = (int64_t)ceilf(ksf + 6.0f * sqrtf(ksf) + 16.0f);
  if (kk == nv || r >= ns) {               // every visible block is a candidate
    if (t == 0) ctr[kThrSlot] = 0u;
    return;
  }
  // this thread's sample keys in registers (ns <= kThrPer * 256 on this path)
  const float* sp = a.samp + (size_t)row * a.samp_ld;
  uint32_t kv[kThrPer];
#pragma unroll
  for (int j = 0; j < kThrPer; j++) {
    const int64_t i = t + (int64_t)j * kFThreads;
    kv[j] = i < ns ? score_key(sp[i]) : 0u;
  }
  uint32_t prefix = 0u, mask = 0u, need = (uint32_t)r;
  const int shs[3] = {21, 10, 0}, wds[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; pass++) {
    const int sh = shs[pass];
    const uint32_t nb = 1u << wds[pass];
    for (int i = t; i < (int)nb; i += blockDim.x) lh[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kThrPer; j++) {
      const int64_t i = t + (int64_t)j * kFThreads;
      if (i < ns && (kv[j] & mask) == prefix) atomicAdd(&lh[(kv[j] >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin(lh, (int)nb, need, tmp, &s_bin, &s_above);
    prefix |= (uint32_t)s_bin << sh;
    mask |= (nb - 1) << sh;
    need -= s_above;
    __syncthreads();                       // s_bin, s_above read by all
  }
  if (t == 0) ctr[kThrSlot] = prefix;      // the r-th largest sample key
}

__global__ void __launch_bounds__(kFThreads) k_select_pf(IndexArgs a) {
  __shared__ uint64_t cl[kEmitCand];
  __shared__ uint32_t bmh[kPfBmWords];     // radix histogram, then the id bitmap
  __shared__ uint32_t tmp[kFThreads / 64];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int kk = (int)(nv < a.k ? nv : a.k);
  int32_t* out = a.topk + (size_t)row * a.k;
  if (kk == nv) {                          // everything visible is selected
    for (int64_t i = t; i < a.k; i += blockDim.x) out[i] = i < nv ? (int32_t)i : -1;
    return;
  }
  uint32_t* ctr = a.ctr + (size_t)row * kCtr;
  const uint32_t n = ctr[kCntSlot];
  const int nw = (int)((nv + 31) / 32);
  if (n < (uint32_t)kk || n > (uint32_t)kCandCap || nw > kPfBmWords) {
    if (t == 0) {                          // the full-score path takes this row
      ctr[kFbSlot] = 1u;
      a.fbl[1 + atomicAdd(&a.fbl[0], 1u)] = (uint32_t)row;
    }
    return;
  }
  for (int i = kk + t; i < a.k; i += blockDim.x) out[i] = -1;
  const uint64_t* cand = a.cand + (size_t)row * kCandCap;
  const bool in_lds = n <= (uint32_t)kEmitCand;
  if (in_lds)
    for (uint32_t i = t; i < n; i += blockDim.x) cl[i] = cand[i];
  // the candidates' common score-key prefix (all are >= the threshold, so
  // usually many top bits agree): the radix passes start below it
  uint32_t k_and = 0xFFFFFFFFu, k_or = 0u;
  for (uint32_t i = t; i < n; i += blockDim.x) {
    const uint32_t k32 = (uint32_t)((in_lds ? cl[i] : cand[i]) >> 32);
    k_and &= k32;
    k_or |= k32;
  }
  __shared__ uint32_t s_and[kFThreads / 64], s_or[kFThreads / 64];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    k_and &= __shfl_xor(k_and, o, 64);
    k_or |= __shfl_xor(k_or, o, 64);
  }
  if ((t & 63) == 0) {
    s_and[t >> 6] = k_and;
    s_or[t >> 6] = k_or;
  }
  __syncthreads();
  k_and = s_and[0] & s_and[1] & s_and[2] & s_and[3];
  k_or = s_or[0] | s_or[1] | s_or[2] | s_or[3];
  const uint32_t diff = k_and ^ k_or;      // bits that differ among the candidates
  const int pbits = diff ? __builtin_clz(diff) : 32;
  const CandSrc src{in_lds ? cl : nullptr, cand, n, nullptr, nv,
                    pbits ? (k_and >> (32 - pbits)) : 0u, pbits, true};
  const uint64_t T = (in_lds && n <= (uint32_t)kRankCand) ? rank_threshold(cl, n, (uint32_t)kk)
                                                          : resolve_threshold(src, (uint32_t)kk, bmh, tmp);
  __syncthreads();                         // the histogram space is free
  for (int i = t; i < nw; i += blockDim.x) bmh[i] = 0u;
  __syncthreads();
  for (uint32_t i = t; i < n; i += blockDim.x) {
    const uint64_t key = in_lds ? cl[i] : cand[i];
    if (key >= T) {
      const uint32_t id = 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu);
      atomicOr(&bmh[id >> 5], 1u << (id & 31));
    }
  }
  __syncthreads();
  // thread t emits bitmap words [t per, (t + 1) per) at its prefix count
  const int per = (nw + kFThreads - 1) / kFThreads;
  const int w0 = t * per, w1 = w0 + per < nw ? w0 + per : nw;
  uint32_t cnt = 0;
  for (int w = w0; w < w1; w++) cnt += (uint32_t)__builtin_popcount(bmh[w]);
  uint32_t pos = block_incl_scan(cnt, tmp) - cnt;
  for (int w = w0; w < w1; w++) {
    uint32_t m = bmh[w];
    while (m) {
      const int bit = __builtin_ctz(m);
      m &= m - 1;
      if (pos < (uint32_t)kk) out[pos] = w * 32 + bit;
      pos++;
    }
  }
}

// ---------------------------------------------------------------- BF16-score selector
// With bf16 scores the two radix digits fix the k-th value T exactly (a bf16
// value's key has its low 16 bits zero), so the selection needs no
// candidate list: every id above T is taken, and of the ids at T the
// lowest-indexed ones, as many as are still needed.

// Second filter: T's digits and, per chunk, its counts above and at T
// (packed: above in the high half, at T in the low half, each <= 4096).
__device__ __forceinline__ void filter2_bf16_row(const IndexArgs& a, const int row) {
  __shared__ uint32_t lh[kBins2];
  __shared__ uint32_t tmp[kFThreads / 64];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  // all global loads first, before the query position arrives
  uint32_t* ctr = a.ctr + (size_t)row * kCtr;
  const uint32_t b1 = ctr[4], above1 = ctr[5];
  constexpr int kPer2 = kBins2 / kFThreads;                          // 8
  const u32x4* gh2 = (const u32x4*)(a.hist2 + (size_t)row * kBins2 + threadIdx.x * kPer2);
  const u32x4 h2a = gh2[0], h2b = gh2[1];
  Group gr;
  issue_group<true>(a, row, blockIdx.x, gr);
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int kk = (int)(nv < a.k ? nv : a.k);
  if (kk == nv || (int64_t)blockIdx.x * kFilterChunk >= nv) return;
  *(u32x4*)&lh[threadIdx.x * kPer2] = h2a;
  *(u32x4*)&lh[threadIdx.x * kPer2 + 4] = h2b;
  __syncthreads();
  find_bin(lh, kBins2, (uint32_t)kk - above1, tmp, &s_bin, &s_above);
  const uint32_t b12 = (b1 << 11) | (uint32_t)s_bin;   // key bits 31..13 of T
  uint32_t k32[kPer];
  const int n_in = finish_group<true>(gr, nv, k32);
  uint32_t above = 0, at = 0;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const bool in = j < n_in;
    const uint32_t d12 = k32[j] >> kSh2;
    above += (in && d12 > b12) ? 1u : 0u;
    at += (in && d12 == b12) ? 1u : 0u;
  }
  const uint32_t packed = block_sum((above << 16) | at, tmp);
  if (threadIdx.x == 0) {
    a.chunk[(size_t)row * n_chunks(a.cap) + blockIdx.x] = packed;
    if (blockIdx.x == 0) {
      ctr[2] = b12;
      ctr[3] = (uint32_t)kk - above1 - s_above;   // ids at T to take
    }
  }
}

__global__ void __launch_bounds__(kFThreads) k_filter2_bf16(IndexArgs a) {
  if (!a.fb_only) {
    filter2_bf16_row(a, (int)blockIdx.y);
    return;
  }
  // the rows the sampled selection handed over, gridDim.y at a time
  const uint32_t n_fb = a.fbl[0];
  for (uint32_t r = blockIdx.y; r < n_fb; r += gridDim.y) {
    filter2_bf16_row(a, (int)a.fbl[1 + r]);
    __syncthreads();
  }
}

// Emit: a workgroup's chunk offset = ids above T in earlier chunks + the ids
// at T taken there; within the chunk one scan of the packed (above, at T)
// counts places every thread's ids; output ascending, tail -1.
__device__ __forceinline__ void emit_bf16_row(const IndexArgs& a, const int row) {
  __shared__ uint32_t tmp[kFThreads / 64];
  const uint32_t* ctr = a.ctr + (size_t)row * kCtr;
  const uint32_t b12 = ctr[2], need = ctr[3];
  const uint32_t* cc = a.chunk + (size_t)row * n_chunks(a.cap);
  const uint32_t cc_first = (int)threadIdx.x < (int)blockIdx.x ? cc[threadIdx.x] : 0u;
  Group gr;
  issue_group<true>(a, row, blockIdx.x, gr);
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int kk = (int)(nv < a.k ? nv : a.k);
  if (kk == nv) return;                    // written by k_filter1
  int32_t* out = a.topk + (size_t)row * a.k;
  if (blockIdx.x == 0)
    for (int i = kk + threadIdx.x; i < a.k; i += blockDim.x) out[i] = -1;
  if ((int64_t)blockIdx.x * kFilterChunk >= nv) return;
  // earlier chunks: ids above T (all taken) and at T (summed separately: the
  // ties may outnumber 16 bits over many chunks)
  uint32_t b_above = cc_first >> 16, b_at = cc_first & 0xFFFFu;
  for (int c = threadIdx.x + blockDim.x; c < (int)blockIdx.x; c += blockDim.x) {
    b_above += cc[c] >> 16;
    b_at += cc[c] & 0xFFFFu;
  }
  b_above = block_sum(b_above, tmp);
  b_at = block_sum(b_at, tmp);
  const uint32_t left = need > b_at ? need - b_at : 0u;   // ties still to take from here on
  uint32_t k32[kPer];
  const int n_in = finish_group<true>(gr, nv, k32);
  const int64_t i0 = gr.g0;
  uint32_t above = 0, at = 0;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const bool in = j < n_in;
    const uint32_t d12 = k32[j] >> kSh2;
    above += (in && d12 > b12) ? 1u : 0u;
    at += (in && d12 == b12) ? 1u : 0u;
  }
  const uint32_t packed = (above << 16) | at;              // chunk sums <= 4096 each
  const uint32_t ex = block_incl_scan(packed, tmp) - packed;
  const uint32_t ex_at = ex & 0xFFFFu;
  uint32_t pos = b_above + (b_at < need ? b_at : need) + (ex >> 16) + (ex_at < left ? ex_at : left);
  uint32_t tie = ex_at;                    // rank of the next id at T within the chunk
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const uint32_t d12 = k32[j] >> kSh2;
    const bool is_at = j < n_in && d12 == b12;
    const bool take = (j < n_in && d12 > b12) || (is_at && tie < left);
    tie += is_at ? 1u : 0u;
    if (take) {
      if (pos < (uint32_t)kk) out[pos] = (int32_t)(i0 + j);
      pos++;
    }
  }
}

__global__ void __launch_bounds__(kFThreads) k_emit_bf16(IndexArgs a) {
  if (!a.fb_only) {
    emit_bf16_row(a, (int)blockIdx.y);
    return;
  }
  // the rows the sampled selection handed over, gridDim.y at a time
  const uint32_t n_fb = a.fbl[0];
  for (uint32_t r = blockIdx.y; r < n_fb; r += gridDim.y) {
    emit_bf16_row(a, (int)a.fbl[1 + r]);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- fixed scratch
// The allocation-free index call carves its workspace out of this array
// instead of a caller's buffer.  Every GPU the library runs on holds its own
// copy (loaded with the code object, kept until the process ends).  Host
// code never passes the array's name to a kernel (on the host it stands for
// a host-side shadow, not a device address): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[kIndexScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t index_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t st, const KernelEvents* ev) {
  const int R = a.B * a.Q;
  if (R == 0) return hipSuccess;
  if (!a.hp_ld) {
    size_t work = (size_t)R * kBins2;
    if (a.key_mx) {
      size_t qthreads = (size_t)R * a.H * 64;
      if (qthreads > work) work = qthreads;
    }
    size_t blocks = (work + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_prep, dim3((unsigned)blocks), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.samp) {
    // sampled-threshold path: sample scan, thresholds, collect scan, exact
    // selection; then the full-score path for the rows it hands over
    const unsigned qt = (unsigned)(a.B * ((a.Q + kQT - 1) / kQT));
    dim3 sgrid(qt, (unsigned)((n_sampled(a.cap) + kQRange - 1) / kQRange));
    dim3 grid(qt, (unsigned)((a.cap + kQRange - 1) / kQRange));
    if (a.score_bf16)
      hipLaunchKernelGGL((k_score_mx_q<kModeSample, true>), sgrid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_score_mx_q<kModeSample, false>), sgrid, dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_thresh, dim3(R), dim3(kFThreads), 0, st, a);
    auto collect = [&](auto kern) {
      if (ev)
        hipExtLaunchKernelGGL(kern, grid, dim3(256), 0, st, ev->start, ev->stop, 0, a);
      else
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, a);
    };
    if (a.score_bf16)
      collect(k_score_mx_q<kModeCollect, true>);
    else
      collect(k_score_mx_q<kModeCollect, false>);
    hipLaunchKernelGGL(k_select_pf, dim3(R), dim3(kFThreads), 0, st, a);
    IndexArgs f = a;
    f.fb_only = 1;
    if (a.score_bf16)
      hipLaunchKernelGGL((k_score_mx_q<kModeStore, true>), grid, dim3(256), 0, st, f);
    else
      hipLaunchKernelGGL((k_score_mx_q<kModeStore, false>), grid, dim3(256), 0, st, f);
    // the handed-over rows, kFbRows at a time
    dim3 fgrid((unsigned)n_chunks(a.cap), (unsigned)(R < kFbRows ? R : kFbRows));
    if (a.score_bf16) {
      hipLaunchKernelGGL(k_filter1<true>, fgrid, dim3(kFThreads), 0, st, f);
      hipLaunchKernelGGL(k_filter2_bf16, fgrid, dim3(kFThreads), 0, st, f);
      hipLaunchKernelGGL(k_emit_bf16, fgrid, dim3(kFThreads), 0, st, f);
    } else {
      hipLaunchKernelGGL(k_filter1<false>, fgrid, dim3(kFThreads), 0, st, f);
      hipLaunchKernelGGL(k_filter2, fgrid, dim3(kFThreads), 0, st, f);
      hipLaunchKernelGGL(k_emit, fgrid, dim3(kFThreads), 0, st, f);
    }
    return hipGetLastError();
  } else if (a.key_mx && a.H == 16 && a.Q >= kQT) {
    dim3 grid((unsigned)(a.B * ((a.Q + kQT - 1) / kQT)),
              (unsigned)((a.cap + kQRange - 1) / kQRange));
    auto store = [&](auto kern) {
      if (ev)
        hipExtLaunchKernelGGL(kern, grid, dim3(256), 0, st, ev->start, ev->stop, 0, a);
      else
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, a);
    };
    if (a.score_bf16)
      store(k_score_mx_q<kModeStore, true>);
    else
      store(k_score_mx_q<kModeStore, false>);
  } else if (a.key_mx) {
    dim3 grid((unsigned)a.score_wgs, R);
    auto go = [&](auto kern) {
      if (ev)
        hipExtLaunchKernelGGL(kern, grid, dim3(64 * kScanWaves), 0, st, ev->start, ev->stop, 0, a);
      else
        hipLaunchKernelGGL(kern, grid, dim3(64 * kScanWaves), 0, st, a);
    };
    const int it = a.score_iters;
    if (a.hp_ld) {
      if (it == 4) go(k_score_mx<true, 4>);
      else if (it == 2) go(k_score_mx<true, 2>);
      else if (it == 1) go(k_score_mx<true, 1>);
      else go(k_score_mx<true, 0>);
    } else {
      if (it == 4) go(k_score_mx<false, 4>);
      else if (it == 2) go(k_score_mx<false, 2>);
      else if (it == 1) go(k_score_mx<false, 1>);
      else go(k_score_mx<false, 0>);
    }
  } else {
    dim3 grid((unsigned)((a.cap + 255) / 256), R);
    size_t smem = sizeof(float) * ((size_t)a.H * a.d + a.H) + sizeof(uint32_t) * kBins1;
    hipLaunchKernelGGL(k_score_f32, grid, dim3(256), smem, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 fgrid((unsigned)n_chunks(a.cap), R);
  if (a.score_bf16)
    hipLaunchKernelGGL(k_filter1<true>, fgrid, dim3(kFThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_filter1<false>, fgrid, dim3(kFThreads), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.score_bf16)
    hipLaunchKernelGGL(k_filter2_bf16, fgrid, dim3(kFThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_filter2, fgrid, dim3(kFThreads), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.elist) return hipSuccess;          // the CSA attention takes the emit step
  if (a.score_bf16)
    hipLaunchKernelGGL(k_emit_bf16, fgrid, dim3(kFThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_emit, fgrid, dim3(kFThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace v4a
