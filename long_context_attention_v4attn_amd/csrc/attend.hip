// Core attention of CSA and HCA: shared-KV MQA over a gathered entry set
// (selected / all visible compressed entries plus the sliding-window raw
// tokens), one joint softmax with an optional per-head sink, split over the
// entry list with a deterministic merge.
//
// Method: [Notes §7] shared key-value MQA (each entry is key AND value), the
// sliding-window branch over the most recent n_win uncompressed entries;
// [Notes §8] compress_ratio table (both sets enter core attention together;
// HCA has no top-k); [Notes §9] attention sink, FP8 KV with BF16 RoPE dims.
//
// Kernels
//   k_attend_fp8  gfx950 MFMA path.  A workgroup = 4 waves = 32 query heads of
//                 one query (two workgroups per compute unit).  The entry
//                 list is walked in tiles of 32 entries staged (raw FP8 codes
//                 + BF16 RoPE + fp32 scale) in LDS once per workgroup:
//                   S = K Q^T   by (entry half, head tile): wave w computes
//                         the complete logits of 16 entries x 16 heads over
//                         all 512 dims with v_mfma_f32_16x16x32_bf16 (K rows
//                         read with ds_read_b128 and widened e4m3 -> bf16
//                         exactly, Q^T in registers);
//                   softmax in those registers (the two waves of a head tile
//                         share a lazily updated running max);
//                   O^T += V^T P^T by dim slice: wave w owns 112 FP8 + 16
//                         RoPE dims for all 32 heads; V^T fragments come
//                         straight from the row-major tile with
//                         ds_read_b64_tr_b8 / _tr_b16 (transpose loads), are
//                         widened once and feed one v_mfma_f32_16x16x32_bf16
//                         per 16-head tile; P^T comes through LDS.
//                 One barrier per tile (three tile buffers, two P buffers).
//                 The per-entry FP8 scale multiplies the non-RoPE logit and
//                 the non-RoPE probability in fp32, so decoding adds no
//                 rounding.  Online softmax in base 2 with a lazily updated
//                 running max (rescale only when the max grows by > 8).
//                 Instantiated with streaming tile loads (one-query CSA
//                 calls: no other reader of the gathered rows) or plain ones
//                 (rows shared by head groups or by a chunk's queries).
//   k_attend_fp8_sel  the same for the fused index + CSA call: the prologue
//                 derives the split's top-k ids from the selector's filter
//                 results (the emit step; see derive_topk) instead of
//                 reading the emitted list.
//   k_attend_fp8_nr  the same with the query RMSNorm + RoPE of the _nr calls
//                 ([Notes §9]) in its prologue: each workgroup normalises and
//                 rotates its 32 heads in registers while its first tiles
//                 load (the per-head sums of squares meet in LDS at the
//                 prologue's first barrier) before the RoPE dims go to LDS;
//                 the output's RoPE dims are rotated back in the epilogue or
//                 the merge.
//   k_attend_f32  fp32 VALU path for unquantised entries (any D <= 512).
//   k_merge_tiled / k_merge  combine split partials in fixed split order.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace v4a {

// ---------------------------------------------------------------- entry list

// Position-dependent sizes of one query's entry list.
struct RowEntries {
  int64_t p;     // query position
  int n_c;       // compressed part length (CSA: k slots; HCA: n_vis)
  int n_w;       // window part length
  int64_t w0;    // first window token
};

__device__ __forceinline__ RowEntries row_entries(const AttendArgs& a, int row) {
  RowEntries r;
  r.p = a.pos[row];
  if (a.csa) {
    r.n_c = a.k;
  } else {
    int64_t nv = r.p < 0 ? 0 : (r.p + 1) / a.m;
    r.n_c = (int)(nv < a.c_cap ? nv : a.c_cap);
  }
  int64_t nw = r.p < 0 ? 0 : (r.p + 1 < a.n_win ? r.p + 1 : a.n_win);
  r.n_w = (int)nw;
  r.w0 = r.p - nw + 1;
  return r;
}

// Source of unified entry e: sets *is_win and returns the cache row, or -1
// when the entry is absent (a top-k slot outside [0, cap)).
__device__ __forceinline__ int64_t entry_source(const AttendArgs& a, const RowEntries& r,
                                                int row, int e, bool* is_win) {
  if (e < r.n_c) {
    *is_win = false;
    if (a.csa) {
      int32_t s = a.topk[(int64_t)row * a.k + e];
      return (s >= 0 && s < a.c_cap) ? (int64_t)s : -1;
    }
    return e;
  }
  *is_win = true;
  int64_t t = r.w0 + (e - r.n_c);
  return t % a.w_cap;
}

// ---------------------------------------------------------------- FP8 MFMA path

constexpr int kTile = 32;                    // entries per tile
constexpr int kNope = 448;                   // FP8 dims
constexpr int kRope = 64;                    // BF16 dims
constexpr int kRowStride = 592;              // LDS row: 448 FP8 + 128 B RoPE + pad
constexpr int kHeads = 32;                   // query heads per workgroup
constexpr int kThreads = 256;                // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;             // lazy max-rescale threshold (log2 units)

// A staged tile: raw e4m3 codes (448 B), bf16 RoPE dims (128 B), the FP8
// scale and an additive mask per entry.
struct __align__(16) Fp8Tile {
  uint8_t rows[kTile * kRowStride];
  float scale[kTile];                      // FP8 scale of the entry (0 if absent)
  float bias[kTile];                       // 0, or -inf for an absent entry
};

// Widen 8 e4m3 codes (two dwords) to 8 bf16 (exact).
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(bf16x8, r);
}

// 4 fp32 -> 4 bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed.
__device__ __forceinline__ u32x2 pack4(const float* v) {
  const bf16x2 lo = {(__bf16)v[0], (__bf16)v[1]};
  const bf16x2 hi = {(__bf16)v[2], (__bf16)v[3]};
  return (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

typedef int v2i_lds __attribute__((ext_vector_type(2)));
typedef short v4s_lds __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_tr8(const uint8_t* p) {
  v2i_lds r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (v2i_lds __attribute__((address_space(3)))*)(p));
  u32x2 o; o[0] = (uint32_t)r[0]; o[1] = (uint32_t)r[1];
  return o;
}

__device__ __forceinline__ u32x2 lds_tr16(const uint8_t* p) {
  v4s_lds r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4s_lds __attribute__((address_space(3)))*)(p));
  u32x2 o;
  o[0] = (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
  o[1] = (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
  return o;
}

// [Notes §9] the output's RoPE dims rotated back by the query position:
// four consecutive dims d0 .. d0+3 (d0 a multiple of 4, two adjacent pairs)
// at RoPE offset r0 = d0 - d_nope >= 0, angle fl32(fl32(p) * inv[pair]).
__device__ __forceinline__ void unrotate4(float* o, const float* inv, int r0, int64_t p) {
  const float pf = (float)p;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    float sn, cs;
    sincos_angle(pf * inv[(r0 >> 1) + j], &sn, &cs);
    const float x0 = o[2 * j], x1 = o[2 * j + 1];
    o[2 * j] = x0 * cs + x1 * sn;          // rotation by -angle
    o[2 * j + 1] = x1 * cs - x0 * sn;
  }
}

// Staging: the 8 threads t = 8e .. 8e+7 move entry e of the tile, so a thread
// resolves one entry's row per tile.  Thread q = t & 7 moves the 16-byte
// chunks q, 8 + q, 16 + q and 24 + q (q < 4) of the FP8 codes, or RoPE chunk
// q - 4 (q >= 4), plus RoPE chunk 4 + (q & 3) and the entry's scale (-1 for
// an absent entry).
struct Stage {
  u32x4 r[5];
  float sc;
};

// Source of every entry of this workgroup's split, resolved once into LDS
// (top-k ids are loaded here, not inside the tile pipeline, so the pipelined
// chunk loads never wait on another global load): >= 0 compressed row,
// -2 - r window ring row r, -1 absent.  Per tile, the kinds of entries it
// holds (bit set), so that a tile of only compressed (only window) rows takes
// a branch-free address path.
constexpr int kMaxSplit = 2048;
constexpr int kMaxTiles = kMaxSplit / kTile + 3;   // + the tiles prefetched past the end
constexpr int kHasComp = 1, kHasWin = 2, kHasAbsent = 4;

// An absent entry (or a slot past the split) reads this row: zero codes and
// RoPE dims, and in place of a scale the marker -1 (cache scales are >= 0),
// which staging turns into scale 0 and mask -inf.
struct __align__(256) AbsentRow {
  uint32_t zero[(kNope + 2 * kRope) / 4];
  float marker;
};
__device__ AbsentRow g_absent = {{}, -1.0f};

// CSA: the top-k id of entry e_beg + threadIdx.x, the workgroup's first load
// (the gather of the first tiles waits on it; the k slots exist whatever the
// query position).  The load is unconditional (a clamped slot, or the
// position array when there is no top-k list) and its value is returned
// as loaded: a load under a branch, or a select on its value, makes the
// compiler wait for it right away.  Only CSA slots e < k use the value.
__device__ __forceinline__ int32_t prefetch_topk(const AttendArgs& a, int row, int e_beg) {
  const int e = e_beg + (int)threadIdx.x;
  const bool has = a.csa && a.k > 0;
  const int32_t* p = has ? a.topk + (int64_t)row * a.k + (e < a.k ? e : a.k - 1)
                         : (const int32_t*)(a.pos + row);
  return *p;
}

// Fused selection ([Notes §7] Top-k; the emit step of the selector moved
// into the attention): the ids of top-k slots e_beg .. e_beg + 255 of the
// row, one per thread, exactly as the emit kernel writes them -- ascending
// ids, lower id first among equal scores, -1 past k' = min(k, n_vis).  The
// threshold T is the need-th largest selection key among the filters'
// candidates (the emit's own resolution); the filters' per-chunk lists hold
// the selection keys of every id at or above the candidates' bin in id
// order, so the ids with key >= T, in list order, are the top-k list.  Head
// group 0 writes its slots to sel_topk (every slot below k belongs to one
// split).  Scratch: the tile buffers' LDS, before the first tile.
constexpr size_t kSelLds = (size_t)kEmitCand * 8 + (size_t)kBinsMax * 4 +
                           (size_t)(kSelMaxChunks + 4) * 4 + (size_t)kThreads * 4 + 16;
constexpr int kSelPer = 16;                  // list entries per thread and step

__device__ int32_t derive_topk(const AttendArgs& a, int row, int hgrp, int e_beg, uint8_t* lds) {
  const int t = threadIdx.x;
  uint64_t* cl = (uint64_t*)lds;                          // candidate keys
  uint32_t* lh = (uint32_t*)(cl + kEmitCand);             // radix histogram
  uint32_t* cstart = lh + kBinsMax;                       // list starts, kSelMaxChunks + 1
  int32_t* slot = (int32_t*)(cstart + kSelMaxChunks + 4);
  uint32_t* tmp = (uint32_t*)(slot + kThreads);
  // Everything that depends on nothing else goes out first, unconditionally
  // (a load under a branch would be waited for at the branch): the query
  // position, the counters, this thread's candidate slot (the list always
  // has kCandCap slots), and the head of one chunk's list: the row's nch
  // chunks (nch <= 256) share the 256 threads, tpc = 256 / nch rounded down
  // to a power of two a chunk, kSelPer entries each (entries past the list
  // are masked below).  When no list is longer than tpc * kSelPer (the
  // 1M-context decode: 64 chunks of about k / 64 entries, 64 loaded each)
  // these are all the entries the selection needs.
  const int64_t p = a.pos[row];
  const uint32_t* ctr = a.sel_ctr + (size_t)row * kCtr;
  const uint32_t n_cand = ctr[0], b12 = ctr[2], need = ctr[3];
  const int64_t nch = n_chunks(a.sel_cap);
  const uint32_t* elen = a.sel_elen + (size_t)row * nch;
  const uint64_t* elist = a.sel_elist + (size_t)row * nch * kFilterChunk;
  const uint64_t* gc = a.sel_cand + (size_t)row * kCandCap;
  const uint64_t c_first = gc[t];
  const int lg = nch <= kThreads ? 32 - __builtin_clz((uint32_t)nch - 1u | 1u) : 0;
  const int tpc = nch <= 1 ? kThreads : (nch <= kThreads ? kThreads >> lg : 1);   // threads a chunk
  const int fc = t / tpc, fq = t % tpc;                   // fast path: chunk, part
  const int64_t fcc = fc < nch ? fc : nch - 1;
  const uint32_t flen = elen[fcc];
  uint64_t key[kSelPer];
  {
    const u32x4* ep = (const u32x4*)(elist + (size_t)fcc * kFilterChunk + fq * kSelPer);
#pragma unroll
    for (int j = 0; j < kSelPer / 2; j++) {
      const u32x4 v = ep[j];
      key[2 * j] = ((uint64_t)v[1] << 32) | v[0];
      key[2 * j + 1] = ((uint64_t)v[3] << 32) | v[2];
    }
  }
  const int64_t nv = n_visible(p, a.sel_m, a.sel_cap);
  const int kk = (int)(nv < a.k ? nv : a.k);
  // every visible block is selected (k_filter1 has written topk)
  if (kk == nv) return e_beg + t < nv ? e_beg + t : -1;
  const int nchv = (int)((nv + kFilterChunk - 1) / kFilterChunk);   // <= kSelMaxChunks
  const bool in_lds = n_cand <= (uint32_t)kEmitCand;
  if (in_lds) {
    if ((uint32_t)t < n_cand) cl[t] = c_first;
    for (uint32_t i = t + kThreads; i < n_cand; i += kThreads) cl[i] = gc[i];
  }
  slot[t] = -1;
  const bool fast = __syncthreads_and(nch <= kThreads &&
                                      (fc >= nchv || flen <= (uint32_t)(tpc * kSelPer)));
  const CandSrc src{in_lds ? cl : nullptr, gc, n_cand, a.sel_scores + (size_t)row * a.sel_sc_ld,
                    nv, b12, 32 - kSh2, n_cand <= (uint32_t)kCandCap};
  const uint64_t T = (src.compact && in_lds && n_cand <= (uint32_t)kRankCand)
                         ? rank_threshold(cl, n_cand, need)
                         : resolve_threshold(src, need, lh, tmp);
  const int r_end = min(e_beg + kThreads, kk);
  if (fast) {
    // the threads in order hold the concatenated lists in order: one scan
    // of the counts of keys >= T places every selected id
    const int nval = fc < nchv ? max(0, min((int)flen - fq * kSelPer, kSelPer)) : 0;
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kSelPer; j++) cnt += (j < nval && key[j] >= T) ? 1u : 0u;
    uint32_t pos = block_incl_scan(cnt, tmp) - cnt;
#pragma unroll
    for (int j = 0; j < kSelPer; j++) {
      if (j < nval && key[j] >= T) {
        if (pos >= (uint32_t)e_beg && pos < (uint32_t)r_end)
          slot[pos - e_beg] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key[j] & 0xFFFFFFFFu));
        pos++;
      }
    }
  } else {
    // general: list starts from the lengths, then walk the concatenated
    // lists kSelPer consecutive entries per thread a step, until this
    // split's slots are placed
    constexpr int kCpt = kSelMaxChunks / kThreads;        // chunks per thread
    uint32_t len[kCpt];
    uint32_t lsum = 0;
#pragma unroll
    for (int j = 0; j < kCpt; j++) {
      const int c = t * kCpt + j;
      len[j] = c < nchv ? elen[c] : 0u;
      lsum += len[j];
    }
    uint32_t n_e;
    uint32_t st = block_incl_scan(lsum, tmp, &n_e) - lsum;
#pragma unroll
    for (int j = 0; j < kCpt; j++) {
      cstart[t * kCpt + j] = st;
      st += len[j];
    }
    if (t == 0) cstart[kSelMaxChunks] = n_e;
    __syncthreads();
    uint32_t done = 0;                     // entries >= T before this step
    for (uint32_t base = 0; base < n_e && done < (uint32_t)r_end; base += kThreads * kSelPer) {
      const uint32_t i0 = base + (uint32_t)t * kSelPer;
      // the chunk of entry i0: the last c < nchv with cstart[c] <= i0
      int c = 0;
      for (int w = kSelMaxChunks / 2; w >= 1; w >>= 1)
        if (c + w < nchv && cstart[c + w] <= i0) c += w;
#pragma unroll
      for (int j = 0; j < kSelPer; j++) {
        const uint32_t i = i0 + j;
        while (c + 1 < nchv && cstart[c + 1] <= i) c++;
        key[j] = i < n_e ? elist[(size_t)c * kFilterChunk + (i - cstart[c])] : 0ull;
      }
      uint32_t cnt = 0;
#pragma unroll
      for (int j = 0; j < kSelPer; j++) cnt += (i0 + j < n_e && key[j] >= T) ? 1u : 0u;
      uint32_t tot;
      uint32_t pos = done + block_incl_scan(cnt, tmp, &tot) - cnt;
#pragma unroll
      for (int j = 0; j < kSelPer; j++) {
        if (i0 + j < n_e && key[j] >= T) {
          if (pos >= (uint32_t)e_beg && pos < (uint32_t)r_end)
            slot[pos - e_beg] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key[j] & 0xFFFFFFFFu));
          pos++;
        }
      }
      done += tot;
    }
  }
  __syncthreads();
  const int32_t id = slot[t];
  if (hgrp == 0 && e_beg + t < a.k) a.sel_topk[(size_t)row * a.k + e_beg + t] = id;
  return id;
}

__device__ __forceinline__ void resolve_sources(const AttendArgs& a, const RowEntries& r, int row,
                                                int e_beg, int n_local, int n_tiles, int32_t pre,
                                                int* src, int* tbits) {
  const int lane = threadIdx.x & 63;
  for (int i = n_tiles + threadIdx.x; i < kMaxTiles; i += blockDim.x) tbits[i] = kHasAbsent;
  // local entry l = base + thread; splits start on tile boundaries, so each
  // half-wave covers one tile and its kinds come from three ballots (slots
  // past the split count as absent)
  for (int base = 0; base < n_tiles * kTile; base += blockDim.x) {
    const int l = base + (int)threadIdx.x;
    int code = -1;
    if (l < n_local) {
      const int e = e_beg + l;
      bool is_win;
      int64_t sr;
      if (a.csa && e < r.n_c && base == 0) {
        is_win = false;                    // the prefetched slot
        sr = (pre >= 0 && pre < a.c_cap) ? (int64_t)pre : -1;
      } else {
        sr = entry_source(a, r, row, e, &is_win);
      }
      // a paged cache: the logical row's pool row ([Notes §11] block table)
      if (a.c_pg.tab && !is_win && sr >= 0) sr = page_row(a.c_pg, row / a.Q, sr);
      code = sr < 0 ? -1 : (is_win ? (int)(-2 - sr) : (int)sr);
      src[l] = code;
    }
    const uint64_t mc = __builtin_amdgcn_ballot_w64(code >= 0);
    const uint64_t mw = __builtin_amdgcn_ballot_w64(code < -1);
    const uint64_t ma = __builtin_amdgcn_ballot_w64(code == -1);
    if ((lane & 31) == 0 && l < n_tiles * kTile) {
      const uint64_t half = lane == 0 ? 0xFFFFFFFFull : 0xFFFFFFFF00000000ull;
      tbits[l / kTile] = ((mc & half) ? kHasComp : 0) | ((mw & half) ? kHasWin : 0) |
                         ((ma & half) ? kHasAbsent : 0);
    }
  }
}

// Per-sequence bases of the compressed cache and the window ring.
struct Bases {
  const uint8_t* cn;
  const uint8_t* cr;
  const float* cs;
  const uint8_t* wn;
  const uint8_t* wr;
  const float* ws;
};

// Every load is issued unconditionally (absent entries read the zero row), so
// the number of loads per tile is fixed and the compiler can keep later
// tiles' loads in flight when it waits for an earlier one.  The address path
// branches on the tile's kind, which is uniform across the workgroup.
// The LDS side of a tile's staging (its kind, this thread's entry source),
// read a step ahead of the loads so that their addresses do not wait on LDS.
struct StageSrc {
  int bits;
  int sraw;
};

__device__ __forceinline__ StageSrc stage_src(const int* src, const int* tbits, int tile) {
  const int le = tile * kTile + ((int)threadIdx.x >> 3);
  StageSrc r;
  r.bits = tbits[tile];
  r.sraw = src[le < kMaxSplit ? le : kMaxSplit - 1];   // always in bounds
  return r;
}

// kStream: streaming (non-temporal) loads, for calls whose rows no other
// workgroup reads again soon (CSA decode: gathered top-k rows of one query);
// otherwise plain loads keep the rows in L2 for the head-group partner and
// the other queries of a chunk.
template <bool kStream>
__device__ __forceinline__ u32x4 tile_load(const uint8_t* p) {
  return kStream ? __builtin_nontemporal_load((const u32x4*)p) : *(const u32x4*)p;
}

template <bool kStream>
__device__ __forceinline__ void stage_load(Bases B, StageSrc ss, int tile, int n_local,
                                           Stage& st) {
  const int t = threadIdx.x;
  const int q = t & 7;
  const int le = tile * kTile + (t >> 3);
  const int bits = __builtin_amdgcn_readfirstlane(ss.bits);
  const uint8_t* nope;
  const uint8_t* rope;
  const float* scp;
  if (bits == kHasComp) {
    const int64_t rr = ss.sraw;
    nope = B.cn + rr * kNope;
    rope = B.cr + rr * (2 * kRope);
    scp = B.cs + rr;
  } else if (bits == kHasWin) {
    const int64_t rr = -2 - ss.sraw;
    nope = B.wn + rr * kNope;
    rope = B.wr + rr * (2 * kRope);
    scp = B.ws + rr;
  } else {
    const int s = le < n_local ? ss.sraw : -1;
    const bool is_win = s < -1;
    const int64_t rr = is_win ? (int64_t)(-2 - s) : (int64_t)s;
    const uint8_t* zero = (const uint8_t*)g_absent.zero;
    if (is_win) {
      nope = B.wn + rr * kNope;
      rope = B.wr + rr * (2 * kRope);
      scp = B.ws + rr;
    } else {
      nope = B.cn + rr * kNope;
      rope = B.cr + rr * (2 * kRope);
      scp = B.cs + rr;
    }
    if (s == -1) {
      nope = zero;
      rope = zero + kNope;
      scp = &g_absent.marker;
    }
  }
  // the values are stored to LDS one step later: using them now would make
  // the compiler wait for these loads immediately
  st.r[0] = tile_load<kStream>(nope + q * 16);
  st.r[1] = tile_load<kStream>(nope + (8 + q) * 16);
  st.r[2] = tile_load<kStream>(nope + (16 + q) * 16);
  st.r[3] = tile_load<kStream>(q < 4 ? nope + (24 + q) * 16 : rope + (q - 4) * 16);
  st.r[4] = tile_load<kStream>(rope + (4 + (q & 3)) * 16);
  st.sc = *scp;
}

// Every value is stored unconditionally (duplicates write identical values),
// so the compiler cannot sink a load into a branch and wait for it there.
__device__ __forceinline__ void stage_store(Fp8Tile* tl, const Stage& st) {
  const int t = threadIdx.x;
  const int e = t >> 3, q = t & 7;
  uint8_t* dst = tl->rows + e * kRowStride;
  *(u32x4*)(dst + q * 16) = st.r[0];
  *(u32x4*)(dst + (8 + q) * 16) = st.r[1];
  *(u32x4*)(dst + (16 + q) * 16) = st.r[2];
  *(u32x4*)(dst + (q < 4 ? (24 + q) * 16 : kNope + (q - 4) * 16)) = st.r[3];
  *(u32x4*)(dst + kNope + (4 + (q & 3)) * 16) = st.r[4];
  tl->scale[e] = st.sc < 0.0f ? 0.0f : st.sc;
  tl->bias[e] = st.sc < 0.0f ? -INFINITY : 0.0f;
}

// Work split of the 4 waves of a workgroup (32 heads of one query):
//  * logits by (entry half, head tile): wave w computes the complete logits
//    S = K Q^T of entries 16 (w & 1) .. +15 x heads 16 (w >> 1) .. +15 of a
//    tile over all 512 dims with v_mfma_f32_16x16x32_bf16 (14 FP8 k-steps,
//    widened exactly, and 2 RoPE k-steps), so no partial logits cross waves;
//  * softmax in the same registers: a lane holds one head (lane & 15) and
//    four entries (4 (lane >> 4) + i) of the wave's half; the two waves of a
//    head tile share the running max through a lazily updated value that
//    both compute identically;
//  * PV by output-dim slice: wave w owns FP8 dims 112w .. 112w+111 and RoPE
//    dims 448 + 16w .. +15 for the 32 heads, so each V^T fragment is widened
//    from FP8 once and feeds two MFMAs (one per 16-head tile); P^T comes
//    through LDS.
// Three tile buffers and two P buffers let one barrier per tile order
// everything: tile t+1 and P(t) are written before it, PV(t) reads after it,
// and a buffer is rewritten only two barriers after its last read.
// A workgroup is small (4 waves, under 80 KB of LDS) so that two run on
// every compute unit and each hides the other's barriers and latencies.
constexpr int kTileBufs = 3;
constexpr int kQrStride = kRope + 8;       // Q RoPE row (bf16): 144 B, conflict-free reads

struct __align__(16) Shared {
  u32x4 pB[2][2][64];                      // P^T operand (RoPE dims) [P buffer][head tile][lane]
  u32x4 pnB[2][2][64];                     // (P * scale)^T operand (FP8 dims)
  float tmx[2][4][16];                     // tile max per head of each wave's entry half
  float alpha[2][kHeads];                  // per-head rescale of a tile (1 = none)
  i32x4 flag[2];                           // a wave's heads outgrew the running max
  uint16_t qr[kHeads][kQrStride];          // Q RoPE dims (bf16) of the 32 heads
  float lsum[4][16];                       // epilogue: each wave's denominators
  float fin[kHeads];                       // per-head output factor (epilogue)
  int tbits[kMaxTiles];                    // entry kinds per tile
};

// Online-softmax state of a lane's head: the running max (identical in the
// 8 lanes x 2 waves that hold a head) and the lane's partial denominator.
struct SoftState {
  float m_run;
  float l_run;
};

// Logits of wave (eh, ht) for tile tl.  MFMA operands: A = K (lane: entry
// 16 eh + (lane & 15), 8 dims of the k-step), B = Q^T (lane: head lane & 15,
// the same dims): lane group g = lane >> 4 takes FP8 dims
// 64 (s >> 1) + 16 g + 8 (s & 1) .. +7 at k-step s < 14 (so a lane reads its
// entry's row in seven 16-byte pieces, and at each k-step the four lane
// groups of a head touch one 64-dim span of Q) and RoPE dims
// 448 + 16 g + 8 (s - 14) .. +7 at s = 14, 15.  The FP8 k-steps' Q^T is
// held in registers, the RoPE k-steps' is read from LDS.  The accumulator value i of a lane is entry 4 (lane >> 4) + i
// of the half, head lane & 15.
__device__ __forceinline__ void qk_tile(const Fp8Tile* tl, const Shared* sh, const bf16x8* qf,
                                        int eh, int ht, int lane, f32x4& sn, f32x4& sr) {
  const int g = lane >> 4;
  const uint8_t* er = tl->rows + (16 * eh + (lane & 15)) * kRowStride;
  // the row is read in two batches (the second in flight under the first
  // batch's MFMAs) to bound the registers held by raw K
  u32x4 kw[7];
#pragma unroll
  for (int j = 0; j < 4; j++) kw[j] = *(const u32x4*)(er + 64 * j + 16 * g);
  __builtin_amdgcn_sched_barrier(0);
  sn = (f32x4){0.f, 0.f, 0.f, 0.f};
  sr = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 4; j < 7; j++) kw[j] = *(const u32x4*)(er + 64 * j + 16 * g);
  const u32x4 kr0 = *(const u32x4*)(er + kNope + 32 * g);
  const u32x4 kr1 = *(const u32x4*)(er + kNope + 32 * g + 16);
  const uint16_t* qrp = &sh->qr[16 * ht + (lane & 15)][16 * g];
  const bf16x8 qr0 = __builtin_bit_cast(bf16x8, *(const u32x4*)qrp);
  const bf16x8 qr1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrp + 8));
#pragma unroll
  for (int j = 0; j < 7; j++) {
    sn = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(kw[j][0], kw[j][1]), qf[2 * j], sn, 0, 0, 0);
    sn = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(kw[j][2], kw[j][3]), qf[2 * j + 1], sn, 0, 0, 0);
  }
  sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr0), qr0, sr, 0, 0, 0);
  sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr1), qr1, sr, 0, 0, 0);
}

// Reductions over the 4 lanes of a head (lane bits 4, 5) without LDS:
// v_permlane16_swap / v_permlane32_swap of a value with itself give each
// lane its own value and that of lane ^ 16 resp. lane ^ 32.  Every lane of a
// head combines the same values, so all four hold identical results.
// (The empty asm statement keeps the compiler from folding the two results
// of a swap into one value.)
template <bool kSwap32>
__device__ __forceinline__ void swap_pair(float v, float& a, float& b) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  auto r = kSwap32 ? __builtin_amdgcn_permlane32_swap(x, x, false, false)
                   : __builtin_amdgcn_permlane16_swap(x, x, false, false);
  uint32_t lo = r[0], hi = r[1];
  __asm__ volatile("" : "+v"(lo), "+v"(hi));
  a = __builtin_bit_cast(float, lo);
  b = __builtin_bit_cast(float, hi);
}

__device__ __forceinline__ float head_max(float v) {
  float a, b;
  swap_pair<false>(v, a, b);
  v = fmaxf(a, b);
  swap_pair<true>(v, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float head_sum(float v) {
  float a, b;
  swap_pair<false>(v, a, b);
  v = a + b;
  swap_pair<true>(v, a, b);
  return a + b;
}

// The lazy-rescale rule: the running max moves only when a tile's max
// exceeds it by more than kRescale (exact: P <= 2^kRescale, and the final
// normalisation uses the same max).
__device__ __forceinline__ bool needs_rescale(float m_run, float tmax) {
  return (m_run == -INFINITY) ? (tmax > -INFINITY) : (tmax > m_run + kRescale);
}

// P and (P * scale) of the lane's four entries against max m (m = -inf:
// nothing seen yet, every logit so far is -inf), written in the PV operand
// layout: head tile ht, lane, slots 4 eh .. +3 (PV's k-slot order: entries
// 4g .. 4g+3 of half 0, then of half 1).  Returns the lane's sum of P.
__device__ __forceinline__ float write_p(Shared* sh, int pb, int ht, int eh, int lane,
                                         const float* s2, f32x4 sc, float m) {
  const float m_use = (m == -INFINITY) ? 0.0f : m;
  float pv[4], pn[4];
  float l = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    // 2^(x) for x <= kRescale; an absent entry gives 2^-inf = 0
    const float p = __builtin_amdgcn_exp2f(s2[i] - m_use);
    l += p;
    pv[i] = p;
    pn[i] = p * sc[i];
  }
  *(u32x2*)((uint8_t*)&sh->pB[pb][ht][lane] + 8 * eh) = pack4(pv);
  *(u32x2*)((uint8_t*)&sh->pnB[pb][ht][lane] + 8 * eh) = pack4(pn);
  return l;
}

// Softmax of the wave's logits, first pass: P against the running max as it
// stands (right unless some wave's tile max outgrows it, which the flags
// report after the barrier; on a split's first tile it always does, so no P
// is written there).  Publishes the wave's tile max per head.
__device__ __forceinline__ float softmax_pass(const Fp8Tile* tl, Shared* sh, const SoftState& S,
                                              f32x4 sn, f32x4 sr, float c2, int pb, int w,
                                              int lane, bool first, float* s2, float& tmax) {
  const int eh = w & 1, ht = w >> 1, g = lane >> 4;
  const f32x4 sc = *(const f32x4*)&tl->scale[16 * eh + 4 * g];
  const f32x4 bi = *(const f32x4*)&tl->bias[16 * eh + 4 * g];
  tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    s2[i] = (sn[i] * sc[i] + sr[i]) * c2 + bi[i];
    tmax = fmaxf(tmax, s2[i]);
  }
  tmax = head_max(tmax);
  const float l = first ? 0.0f : write_p(sh, pb, ht, eh, lane, s2, sc, S.m_run);
  if (lane < 16) sh->tmx[pb][w][lane] = tmax;
  const int any = __builtin_amdgcn_ballot_w64(needs_rescale(S.m_run, tmax)) != 0;
  if (lane == 0) sh->flag[pb][w] = any;
  return l;
}

// Output dims of PV wave w, block db (16 dims): FP8 dims 112w + 16db for
// db < 7, RoPE dims 448 + 16w for db = 7 -- every wave the same mix, so the
// PV code has no branches on the wave.
__device__ __forceinline__ int pv_dim0(int w, int db) { return db < 7 ? 112 * w + 16 * db : kNope + 16 * w; }

// PV for wave `ds`, both head groups: acc[db][ht] = O^T block of dims
// pv_dim0(ds, db) .. +16 x heads 16ht .. +16.  FP8 blocks: 8-bit transpose
// reads, widened, times (P * scale)^T; the RoPE block: 16-bit transpose
// reads times P^T.  The V^T reads depend only on the tile, so they are
// issued right after the barrier, together with the rescale flags, and
// their latency covers the flags' (pv_load); P^T is read after the (rare)
// rescale step has settled it (pv_mma).
struct VFrag {
  u32x2 w8[7];                             // FP8 blocks, raw codes
  u32x2 lo, hi;                            // RoPE block, bf16
};

__device__ __forceinline__ VFrag pv_load(const Fp8Tile* tl, int ds, int g, int li) {
  // lane group g's k-values are entries {4g..4g+3, 16+4g..16+4g+3}; source
  // lane s of the group points at entry k = s/2 (tr8) resp. s/4 (tr16)
  const int s = li;
  const int kk8 = s >> 1;
  const int ent8 = (kk8 < 4) ? (g * 4 + kk8) : (16 + g * 4 + kk8 - 4);
  const uint8_t* vb8 = tl->rows + ent8 * kRowStride + (s & 1) * 8 + ds * 112;
  VFrag v;
#pragma unroll
  for (int db = 0; db < 7; db++) v.w8[db] = lds_tr8(vb8 + db * 16);
  const int kk16 = s >> 2;
  const uint8_t* vlo = tl->rows + (g * 4 + kk16) * kRowStride + kNope + ds * 32 + (s & 3) * 8;
  const uint8_t* vhi = tl->rows + (16 + g * 4 + kk16) * kRowStride + kNope + ds * 32 + (s & 3) * 8;
  v.lo = lds_tr16(vlo);
  v.hi = lds_tr16(vhi);
  return v;
}

__device__ __forceinline__ void pv_mma(const Shared* sh, f32x4 (*acc)[2], const VFrag& vf, int li,
                                       int pb, bool rescale) {
  const int lane = threadIdx.x & 63;
  const bf16x8 pn0 = __builtin_bit_cast(bf16x8, sh->pnB[pb][0][lane]);
  const bf16x8 pn1 = __builtin_bit_cast(bf16x8, sh->pnB[pb][1][lane]);
  const bf16x8 pb0 = __builtin_bit_cast(bf16x8, sh->pB[pb][0][lane]);
  const bf16x8 pb1 = __builtin_bit_cast(bf16x8, sh->pB[pb][1][lane]);
  if (rescale) {
#pragma unroll
    for (int ht = 0; ht < 2; ht++) {
      const float al = sh->alpha[pb][ht * 16 + li];
#pragma unroll
      for (int db = 0; db < 8; db++) acc[db][ht] *= al;
    }
  }
#pragma unroll
  for (int db = 0; db < 7; db++) {
    const bf16x8 v = widen8(vf.w8[db][0], vf.w8[db][1]);
    acc[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pn0, acc[db][0], 0, 0, 0);
    acc[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pn1, acc[db][1], 0, 0, 0);
  }
  const bf16x8 vr = __builtin_bit_cast(bf16x8, (u32x4){vf.lo[0], vf.lo[1], vf.hi[0], vf.hi[1]});
  acc[7][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr, pb0, acc[7][0], 0, 0, 0);
  acc[7][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr, pb1, acc[7][1], 0, 0, 0);
}

// Workgroup -> (query row, split, group of 32 heads).  Workgroups are
// dispatched to the 8 XCDs round-robin; consecutive positions within one XCD
// take the head groups, then the splits, of one query, so the workgroups
// that read the same tiles share an XCD (its L2).
__device__ __forceinline__ bool wg_coords(const AttendArgs& a, int* row, int* split, int* hgrp) {
  const int n_hg = (a.H + kHeads - 1) / kHeads;
  const int64_t N = (int64_t)a.B * a.Q * n_hg * a.n_split;
  const int64_t per = (N + 7) / 8;
  const int64_t L = blockIdx.x;
  const int64_t P = (L % 8) * per + L / 8;
  if (P >= N) return false;
  *hgrp = (int)(P % n_hg);
  const int64_t rest = P / n_hg;
  *split = (int)(rest % a.n_split);
  *row = (int)(rest / a.n_split);
  return true;
}

// Split partials of the FP8 path live in the workspace in the accumulator
// layout, so that a wave stores (and the merge loads) whole contiguous runs:
// the block of (row, split, head group) holds nh x 512 values ordered
// [PV wave 4][dim block 8][head tile nht][lane 64][4] (dims: pv_dim0).
__device__ __forceinline__ int64_t part_block(const AttendArgs& a, int row, int split, int hgrp) {
  return (((int64_t)row * a.n_split + split) * a.H + hgrp * kHeads) * (kNope + kRope);
}

// kNr: the _nr calls' query RMSNorm + RoPE ([Notes §9]) fused into the
// prologue (see below); the output's rotation back is in the epilogues.
template <bool kNr, bool kStream, bool kSel = false>
__device__ __forceinline__ void attend_fp8(AttendArgs a) {
  __shared__ Fp8Tile tiles[kTileBufs];
  __shared__ Shared sh;
  __shared__ int src[kMaxSplit];
  int row, split, hgrp;
  if (!wg_coords(a, &row, &split, &hgrp)) return;
  int32_t pre = kSel ? -1 : prefetch_topk(a, row, split * a.split_size);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int eh = wave & 1, wht = wave >> 1;  // logits: entry half, head tile
  const int b = row / a.Q;
  const int g = lane >> 4;                 // PV: lane group 0..3
  const int li = lane & 15;
  const int nht = min(2, (a.H - hgrp * kHeads) / 16);   // head tiles present (H % 16 == 0)
  const int D = kNope + kRope;

  // Q^T fragments of head 16 wht + (lane & 15) (MFMA B operand), loaded
  // right after the top-k ids (they depend on nothing): k-step s < 14 holds
  // FP8 dims 64 (s >> 1) + 16 g + 8 (s & 1) .. +7 (zero for heads beyond
  // H); the RoPE dims go to LDS
  bf16x8 qf[14];
  {
    const int qh = hgrp * kHeads + 16 * wht + li;
    const bool q_ok = qh < a.H;
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)row * a.H + (q_ok ? qh : 0)) * D;
#pragma unroll
    for (int s = 0; s < 14; s++) {
      u32x4 v = *(const u32x4*)(qp + 64 * (s >> 1) + 16 * g + 8 * (s & 1));
      if (!q_ok) v = (u32x4){0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // RoPE dims of the 32 heads, 16 bytes per thread: loaded now, stored to
  // LDS once the first tiles' loads are out (so that waiting for this load
  // holds back neither source resolution nor the gather)
  // (an unconditional load: a conditional one would make the compiler wait
  // for it, and for the loads before it, where the branches join)
  const int rh = threadIdx.x >> 3, rc = threadIdx.x & 7;
  const bool r_ok = hgrp * kHeads + rh < a.H;
  u32x4 qrv = *(const u32x4*)((const uint16_t*)a.q +
                              ((int64_t)row * a.H + (r_ok ? hgrp * kHeads + rh : 0)) * D + kNope + 8 * rc);
  if (!r_ok) qrv = (u32x4){0u, 0u, 0u, 0u};
  // _nr: the norm weights (two per thread), the RoPE inverse frequencies of
  // this thread's four pairs and the query position, loaded with the query
  // (unconditional loads; a missing weight or table reads the query instead)
  float2 gam = {1.0f, 1.0f};
  f32x4 ivf = {0.0f, 0.0f, 0.0f, 0.0f};
  int64_t p_q = 0;
  if (kNr) {
    gam = *(const float2*)(a.nr_gamma ? a.nr_gamma + 2 * threadIdx.x : (const float*)a.q);
    ivf = *(const f32x4*)(a.nr_inv ? a.nr_inv + 4 * rc : (const float*)a.q);
    p_q = a.pos[row];
  }
  const int e_beg = split * a.split_size;
  // fused selection: the split's top-k ids (the tile buffers are free
  // until the first tile is staged, after the barrier below); called before
  // the entry list's sizes are read, so that its loads go out with the
  // query position's rather than one round trip after it
  if (kSel && e_beg < a.k) pre = derive_topk(a, row, hgrp, e_beg, (uint8_t*)tiles);
  const RowEntries r = row_entries(a, row);
  const int n_tot = r.n_c + r.n_w;
  const int e_end = min(e_beg + a.split_size, n_tot);
  // uniform across the workgroup: kept in scalar registers so that the tile
  // loop's branches are scalar
  const int n_local = __builtin_amdgcn_readfirstlane(e_end > e_beg ? e_end - e_beg : 0);
  const int n_tiles = (n_local + kTile - 1) / kTile;
  resolve_sources(a, r, row, e_beg, n_local, n_tiles, pre, src, sh.tbits);
  if (kNr) {
    // the weights go to the third tile buffer (first written after the
    // loop's first barrier); each head's sum of squares in two parts: its
    // FP8 dims over the four lane groups that hold them (fin), its RoPE dims
    // over the eight threads that hold them (lsum; both are epilogue slots)
    *(float2*)((float*)tiles[2].rows + 2 * threadIdx.x) = gam;
    float sq = 0.0f;
#pragma unroll
    for (int s = 0; s < 14; s++) {
      const u32x4 w = __builtin_bit_cast(u32x4, qf[s]);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float x0 = bf16_bits_to_f32(w[i] & 0xFFFFu), x1 = bf16_bits_to_f32(w[i] >> 16);
        sq += x0 * x0 + x1 * x1;
      }
    }
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    if (eh == 0 && g == 0) sh.fin[16 * wht + li] = sq;
    float rq = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float x0 = bf16_bits_to_f32(qrv[i] & 0xFFFFu), x1 = bf16_bits_to_f32(qrv[i] >> 16);
      rq += x0 * x0 + x1 * x1;
    }
    rq += __shfl_xor(rq, 1, 64);
    rq += __shfl_xor(rq, 2, 64);
    rq += __shfl_xor(rq, 4, 64);
    if (rc == 0) (&sh.lsum[0][0])[rh] = rq;
  }
  __syncthreads();

  Bases B;
  const int64_t cbase = a.c_pg.tab ? 0 : (int64_t)b * a.c_cap;   // paged: pool rows
  B.cn = a.c_nope + cbase * kNope;
  B.cr = (const uint8_t*)(a.c_rope + cbase * kRope);
  B.cs = a.c_scale + cbase;
  B.wn = a.w_nope + (int64_t)b * a.w_cap * kNope;
  B.wr = (const uint8_t*)(a.w_rope + (int64_t)b * a.w_cap * kRope);
  B.ws = a.w_scale + (int64_t)b * a.w_cap;

  // one tile in flight in registers while another is computed (a second
  // register set would push the kernel past 256 VGPRs into scratch); every
  // stage_load issues the same loads (tiles past the split read the zero row)
  Stage st;
  stage_load<kStream>(B, stage_src(src, sh.tbits, 0), 0, n_local, st);

  f32x4 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  SoftState S;
  S.m_run = -INFINITY;
  S.l_run = 0.0f;
  const float c2 = a.sm_scale * kLog2e;

  // (_nr: the query's norm and rotation run while the first tiles load)
  if (kNr) {
    // x * r * gamma with r = 1 / sqrt(mean(x^2) + eps) over the head's 512
    // dims, then the RoPE dims' adjacent pairs rotated by the query
    // position; the results are rounded to bf16 once, as the operands
    const float* gl = (const float*)tiles[2].rows;
    const float* sql = &sh.lsum[0][0];
    if (a.nr_gamma) {
      const int hq = 16 * wht + li;
      const float rn = 1.0f / sqrtf((sh.fin[hq] + sql[hq]) / (float)D + a.nr_eps);
#pragma unroll
      for (int s = 0; s < 14; s++) {
        const u32x4 w = __builtin_bit_cast(u32x4, qf[s]);
        const float* gd = gl + 64 * (s >> 1) + 16 * g + 8 * (s & 1);
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu) * rn * gd[2 * i];
          x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16) * rn * gd[2 * i + 1];
        }
        const u32x2 lo = pack4(x), hi = pack4(x + 4);
        qf[s] = __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], hi[0], hi[1]});
      }
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      x[2 * i] = bf16_bits_to_f32(qrv[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_bits_to_f32(qrv[i] >> 16);
    }
    if (a.nr_gamma) {
      const float rr = 1.0f / sqrtf((sh.fin[rh] + sql[rh]) / (float)D + a.nr_eps);
#pragma unroll
      for (int i = 0; i < 8; i++) x[i] = x[i] * rr * gl[kNope + 8 * rc + i];
    }
    if (a.nr_inv) {
      const float pf = (float)p_q;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        float sn, cs;
        sincos_angle(pf * ivf[j], &sn, &cs);
        const float x0 = x[2 * j], x1 = x[2 * j + 1];
        x[2 * j] = x0 * cs - x1 * sn;
        x[2 * j + 1] = x0 * sn + x1 * cs;
      }
    }
    const u32x2 lo = pack4(x), hi = pack4(x + 4);
    qrv = (u32x4){lo[0], lo[1], hi[0], hi[1]};
  }
  stage_store(&tiles[0], st);
  stage_load<kStream>(B, stage_src(src, sh.tbits, 1), 1, n_local, st);
  *(u32x4*)&sh.qr[rh][8 * rc] = qrv;
  __syncthreads();

  // step t (tile t in buffer cb, P buffer pb = t & 1): logits and softmax
  // of tile t in registers, P(t) and tile t+1 (buffer nb) into LDS, the
  // register set refilled with tile t+2 | barrier | PV of tile t.  When a
  // wave's tile max outgrew the running max (and on the first tile), the
  // two waves of each head tile agree on the tile max through LDS, P(t) is
  // (re)written against the new max and a second barrier publishes it and
  // the rescale factors.  Unrolled by two so that the P buffers alternate
  // statically.
  auto step = [&](int t, int cb, int nb, int pb, Stage& nxt) {
    const StageSrc ns = stage_src(src, sh.tbits, t + 2);
    f32x4 sn, sr;
    float s2[4], tmax;
    // A wave's logits and softmax run at raised issue priority, so that the
    // MFMA chain and the softmax that waits on it are not interleaved with
    // the other wave's staging and PV on the same SIMD (HCA decode attention
    // 40.4 -> 39.0 us); one-query CSA calls (streaming loads) showed no gain
    // and keep the default.
    if (!kStream) __builtin_amdgcn_s_setprio(1);
    qk_tile(&tiles[cb], &sh, qf, eh, wht, lane, sn, sr);
    const bool first = t == 0;
    float l_add = softmax_pass(&tiles[cb], &sh, S, sn, sr, c2, pb, wave, lane, first, s2, tmax);
    if (!kStream) __builtin_amdgcn_s_setprio(0);
    stage_store(&tiles[nb], nxt);
    stage_load<kStream>(B, ns, t + 2, n_local, nxt);
    __syncthreads();
    VFrag vf = pv_load(&tiles[cb], wave, g, li);
    const i32x4 fl = sh.flag[pb];
    const bool rescale = first || ((fl[0] | fl[1]) | (fl[2] | fl[3])) != 0;
    if (rescale) {
      // max over both entry halves, in the same order in both waves
      const float tp = sh.tmx[pb][wave ^ 1][li];
      const float tj = eh == 0 ? fmaxf(tmax, tp) : fmaxf(tp, tmax);
      float alpha = 1.0f;
      if (needs_rescale(S.m_run, tj)) {
        alpha = (S.m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(S.m_run - tj);
        S.l_run *= alpha;
        S.m_run = tj;
      }
      const f32x4 sc = *(const f32x4*)&tiles[cb].scale[16 * eh + 4 * g];
      l_add = write_p(&sh, pb, wht, eh, lane, s2, sc, S.m_run);
      // (the four lanes of a head hold the same factor and all store it)
      if (eh == 0) sh.alpha[pb][16 * wht + li] = alpha;
      __syncthreads();
      // read again rather than held across this rare path (register room)
      vf = pv_load(&tiles[cb], wave, g, li);
    }
    S.l_run += l_add;
    pv_mma(&sh, acc, vf, li, pb, rescale);
  };
  int t = 0, cb = 0;
  for (; t + 1 < n_tiles; t += 2) {
    const int nb = cb == kTileBufs - 1 ? 0 : cb + 1;
    const int nb2 = nb == kTileBufs - 1 ? 0 : nb + 1;
    step(t, cb, nb, 0, st);
    step(t + 1, nb, nb2, 1, st);
    cb = nb2;
  }
  if (t < n_tiles) step(t, cb, cb == kTileBufs - 1 ? 0 : cb + 1, 0, st);

  // ---- epilogue: each wave's denominators per head (summed over its four
  // lane groups), then the two entry halves added in fixed order by the
  // lanes of the half-0 wave, which publish each head's factor
  const float l_w = head_sum(S.l_run);
  if (lane < 16) sh.lsum[wave][lane] = l_w;
  __syncthreads();
  if (eh == 0 && lane < 16) {
    const float l_tot = sh.lsum[wave][lane] + sh.lsum[wave + 1][lane];
    const int jh = 16 * wht + lane;
    const int head = hgrp * kHeads + jh;
    const bool head_ok = head < a.H;
    float f;
    if (a.n_split == 1) {
      const float z2 = (a.sink && head_ok) ? a.sink[head] * kLog2e : -INFINITY;
      const float M = fmaxf(S.m_run, z2);
      const float so = (S.m_run == -INFINITY) ? 0.0f : exp2f(S.m_run - M);
      const float den = l_tot * so + ((z2 == -INFINITY) ? 0.0f : exp2f(z2 - M));
      f = den > 0.0f ? so / den : 0.0f;
    } else {
      // partial: O / l (zero when the split saw nothing) + (max, denominator)
      f = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      if (head_ok) {
        const int64_t pi = ((int64_t)row * a.n_split + split) * a.H + head;
        a.part_ml[pi * 2 + 0] = l_tot > 0.0f ? S.m_run : -INFINITY;
        a.part_ml[pi * 2 + 1] = l_tot;
      }
    }
    sh.fin[jh] = f;
  }
  __syncthreads();
  // PV wave `wave` holds O^T dims pv_dim0(wave, db) + 4g + i of head 16ht + li
  if (a.n_split == 1) {
#pragma unroll
    for (int ht = 0; ht < 2; ht++) {
      if (ht >= nht) break;
      const float f = sh.fin[ht * 16 + li];
      const int64_t ob = ((int64_t)row * a.H + hgrp * kHeads + ht * 16 + li) * D + g * 4;
#pragma unroll
      for (int db = 0; db < 8; db++) {
        f32x4 o = acc[db][ht] * f;
        if (db == 7 && a.nr_inv) {
          // the RoPE block: dims 448 + 16 wave + 4g .. +3
          float ov[4] = {o[0], o[1], o[2], o[3]};
          unrotate4(ov, a.nr_inv, 16 * wave + 4 * g, a.pos[row]);
          o = (f32x4){ov[0], ov[1], ov[2], ov[3]};
        }
        const int64_t oi = ob + pv_dim0(wave, db);
        if (a.out_bf16) {
          const float ov[4] = {o[0], o[1], o[2], o[3]};
          __builtin_nontemporal_store(pack4(ov), (u32x2*)((uint16_t*)a.out + oi));
        } else {
          *(f32x4*)((float*)a.out + oi) = o;
        }
      }
    }
  } else {
    uint16_t* po = (uint16_t*)a.part_o + part_block(a, row, split, hgrp);
#pragma unroll
    for (int db = 0; db < 8; db++) {
#pragma unroll
      for (int ht = 0; ht < 2; ht++) {
        if (ht >= nht) break;
        const f32x4 o = acc[db][ht] * sh.fin[ht * 16 + li];
        const float ov[4] = {o[0], o[1], o[2], o[3]};
        // streaming stores: the merge reads them once, and lines that do
        // not sit dirty in L2 need no write-back when the kernel ends
        __builtin_nontemporal_store(pack4(ov),
                                    (u32x2*)(po + (((int64_t)(wave * 8 + db) * nht + ht) * 64 + lane) * 4));
      }
    }
  }
}

template <bool kStream>
__global__ void __launch_bounds__(kThreads, 2) k_attend_fp8(AttendArgs a) { attend_fp8<false, kStream>(a); }
template <bool kStream>
__global__ void __launch_bounds__(kThreads, 2) k_attend_fp8_nr(AttendArgs a) { attend_fp8<true, kStream>(a); }
template <bool kStream>
__global__ void __launch_bounds__(kThreads, 2) k_attend_fp8_sel(AttendArgs a) {
  attend_fp8<false, kStream, true>(a);
}
static_assert(kSelLds <= sizeof(Fp8Tile) * kTileBufs, "the fused selection's scratch fits the tile buffers");

// ---------------------------------------------------------------- fp32 VALU path
// One workgroup per (query, split, head group of kF32Heads); entries are
// processed in chunks of kF32Chunk staged in LDS; every thread owns a fixed
// set of (head, dim) outputs.  Plain fp32 arithmetic throughout.

constexpr int kF32Chunk = 16;

__global__ void __launch_bounds__(256) k_attend_f32(AttendArgs a) {
  extern __shared__ float sm[];
  const int row = blockIdx.x, split = blockIdx.y, hg = blockIdx.z;
  const int b = row / a.Q;
  const int D = a.d_nope + a.d_rope;
  const int h0 = hg * a.f32_heads;
  const int nh = min(a.f32_heads, a.H - h0);
  float* ent = sm;                                  // [kF32Chunk][D]
  float* qs = ent + kF32Chunk * D;                  // [nh][D]
  float* lg = qs + a.f32_heads * D;                 // [nh][kF32Chunk]
  float* mrun = lg + a.f32_heads * kF32Chunk;       // [nh]
  float* lrun = mrun + a.f32_heads;                 // [nh]
  float* alph = lrun + a.f32_heads;                 // [nh]
  int* vld = (int*)(alph + a.f32_heads);            // [kF32Chunk]

  RowEntries r = row_entries(a, row);
  const int n_tot = r.n_c + r.n_w;
  const int e_beg = split * a.split_size;
  const int e_end = min(e_beg + a.split_size, n_tot);

  for (int i = threadIdx.x; i < nh * D; i += blockDim.x) {
    int h = i / D, d = i % D;
    qs[i] = load_as_f32(a.q, a.q_bf16, ((int64_t)row * a.H + h0 + h) * D + d);
  }
  for (int h = threadIdx.x; h < nh; h += blockDim.x) { mrun[h] = -INFINITY; lrun[h] = 0.f; }
  // outputs owned by this thread: (h, d) = idx / D, idx % D for idx = t + k*256
  constexpr int kMaxOut = 32;
  float o[kMaxOut];
#pragma unroll
  for (int j = 0; j < kMaxOut; j++) o[j] = 0.f;
  const float c2 = a.sm_scale * kLog2e;
  __syncthreads();

  for (int c0 = e_beg; c0 < e_end; c0 += kF32Chunk) {
    const int nc = min(kF32Chunk, e_end - c0);
    // stage entries
    for (int i = threadIdx.x; i < kF32Chunk * D; i += blockDim.x) {
      int e = i / D, d = i % D;
      float v = 0.f;
      int ok = 0;
      if (e < nc) {
        bool is_win;
        int64_t src = entry_source(a, r, row, c0 + e, &is_win);
        if (src >= 0) {
          const float* nope = (const float*)(is_win ? (const void*)a.w_nope : (const void*)a.c_nope);
          const float* rope = (const float*)(is_win ? (const void*)a.w_rope : (const void*)a.c_rope);
          int64_t cap = is_win ? a.w_cap : a.c_cap;
          int64_t ri = (int64_t)b * cap + src;
          v = d < a.d_nope ? nope[ri * a.d_nope + d] : rope[ri * a.d_rope + (d - a.d_nope)];
          ok = 1;
        }
      }
      ent[i] = v;
      if (d == 0) vld[e] = ok;
    }
    __syncthreads();
    // logits
    for (int i = threadIdx.x; i < nh * kF32Chunk; i += blockDim.x) {
      int h = i / kF32Chunk, e = i % kF32Chunk;
      float s = 0.f;
      for (int d = 0; d < D; d++) s += qs[h * D + d] * ent[e * D + d];
      lg[i] = (e < nc && vld[e]) ? s * c2 : -INFINITY;
    }
    __syncthreads();
    // online softmax bookkeeping per head
    for (int h = threadIdx.x; h < nh; h += blockDim.x) {
      float mx = -INFINITY;
      for (int e = 0; e < kF32Chunk; e++) mx = fmaxf(mx, lg[h * kF32Chunk + e]);
      float m_new = fmaxf(mrun[h], mx);
      float m_use = m_new == -INFINITY ? 0.f : m_new;
      float al = mrun[h] == -INFINITY ? 0.f : exp2f(mrun[h] - m_use);
      float ls = 0.f;
      for (int e = 0; e < kF32Chunk; e++) {
        float p = exp2f(lg[h * kF32Chunk + e] - m_use);
        lg[h * kF32Chunk + e] = p;
        ls += p;
      }
      lrun[h] = lrun[h] * al + ls;
      mrun[h] = m_new;
      alph[h] = al;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxOut; j++) {
      int idx = threadIdx.x + j * blockDim.x;
      if (idx < nh * D) {
        int h = idx / D, d = idx % D;
        float acc = o[j] * alph[h];
        for (int e = 0; e < kF32Chunk; e++) acc += lg[h * kF32Chunk + e] * ent[e * D + d];
        o[j] = acc;
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < kMaxOut; j++) {
    int idx = threadIdx.x + j * blockDim.x;
    if (idx >= nh * D) continue;
    int h = idx / D, d = idx % D;
    int head = h0 + h;
    if (a.n_split == 1) {
      float z2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
      float m = mrun[h];
      float M = fmaxf(m, z2);
      float so = m == -INFINITY ? 0.f : exp2f(m - M);
      float den = lrun[h] * so + (z2 == -INFINITY ? 0.f : exp2f(z2 - M));
      float v = den > 0.f ? o[j] * so / den : 0.f;
      int64_t oi = ((int64_t)row * a.H + head) * D + d;
      if (a.out_bf16) ((uint16_t*)a.out)[oi] = (uint16_t)f32_to_bf16_bits(v);
      else ((float*)a.out)[oi] = v;
    } else {
      // partial: O / l in fp32 (zero when the split saw nothing) + (max, denominator)
      int64_t pi = ((int64_t)row * a.n_split + split) * a.H + head;
      const float l = lrun[h];
      ((float*)a.part_o)[pi * D + d] = l > 0.f ? o[j] / l : 0.f;
      if (d == 0) {
        a.part_ml[pi * 2] = l > 0.f ? mrun[h] : -INFINITY;
        a.part_ml[pi * 2 + 1] = l;
      }
    }
  }
}

// ---------------------------------------------------------------- merge
// Split s carries On_s = O_s / l_s and (m_s, l_s).  With M = max(max_s m_s, z):
//   out = sum_s w_s On_s / (sum_s w_s + 2^(z - M)),  w_s = l_s 2^(m_s - M),
// splits visited in index order (deterministic).  fp32 path: row-major fp32
// partials; one workgroup per (query, 4 heads); each thread owns 8
// consecutive dims of one head.
constexpr int kMergeHeads = 4;

__global__ void __launch_bounds__(256) k_merge(AttendArgs a) {
  const int row = blockIdx.x;
  const int D = a.d_nope + a.d_rope;
  const int per_head = D / 8;                        // threads per head
  const int hl = threadIdx.x / per_head;
  const int d0 = (threadIdx.x % per_head) * 8;
  const int head = blockIdx.y * kMergeHeads + hl;
  if (hl >= kMergeHeads || head >= a.H) return;
  const float* ml = a.part_ml + ((int64_t)row * a.n_split * a.H) * 2;
  const float z2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
  float M = z2;
  for (int s = 0; s < a.n_split; s++) M = fmaxf(M, ml[((int64_t)s * a.H + head) * 2]);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; i++) acc[i] = 0.f;
  float den = (M == -INFINITY || z2 == -INFINITY) ? 0.f : exp2f(z2 - M);
  for (int s = 0; s < a.n_split; s++) {
    const float m = ml[((int64_t)s * a.H + head) * 2];
    if (m == -INFINITY) continue;
    const float w = ml[((int64_t)s * a.H + head) * 2 + 1] * exp2f(m - M);
    den += w;
    const float* p = (const float*)a.part_o + (((int64_t)row * a.n_split + s) * a.H + head) * D + d0;
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] += w * p[i];
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  const int64_t oi = ((int64_t)row * a.H + head) * D + d0;
  if (a.out_bf16) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; i++)
      v[i] = f32_to_bf16_bits(acc[2 * i] * inv) | (f32_to_bf16_bits(acc[2 * i + 1] * inv) << 16);
    *(u32x4*)((uint16_t*)a.out + oi) = v;
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) ((float*)a.out)[oi + i] = acc[i] * inv;
  }
}

// FP8 path: partials in the accumulator layout (bf16).  One workgroup per
// (query, head group of 32, 1/64 of the block): 64 groups of 4 consecutive
// values (4 dims of one head) x 4 split phases; phase p takes the splits
// s = p, p + 4, ... and the phases combine their maxima, then their weighted
// sums, through LDS in fixed order (deterministic).
constexpr int kMergePhases = 4;
constexpr int kMergeRegs = 8;              // splits per phase held in registers

__global__ void __launch_bounds__(256) k_merge_tiled(AttendArgs a) {
  __shared__ float red[kMergePhases][64][6];
  const int row = blockIdx.x, hgrp = blockIdx.y;
  const int D = kNope + kRope;
  const int nht = min(2, (a.H - hgrp * kHeads) / 16);
  const int n_vals = nht * 16 * D;                     // values in the block
  const int vg = threadIdx.x & 63, ph = threadIdx.x >> 6;
  const int j = (blockIdx.z * 64 + vg) * 4;            // first owned value
  const bool active = j < n_vals;
  // decode [dim slice][dim block][head tile][lane][4]
  const int q4 = (active ? j : 0) >> 2;
  const int ln = q4 & 63;
  const int ht = (q4 >> 6) % nht;
  const int sb = (q4 >> 6) / nht;                      // PV wave * 8 + dim block
  const int head = hgrp * kHeads + ht * 16 + (ln & 15);
  const int d0 = pv_dim0(sb >> 3, sb & 7) + (ln >> 4) * 4;
  const f32x2* ml = (const f32x2*)a.part_ml + (int64_t)row * a.n_split * a.H + head;
  // (an inactive thread reads the block's first values: always in bounds)
  const uint16_t* po = (const uint16_t*)a.part_o + part_block(a, row, 0, hgrp) + (active ? j : 0);
  const int64_t sstride = (int64_t)a.H * D;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  float M = -INFINITY;
  const float z2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
  // the output rotation's inputs, loaded with the rest (used when nr_inv is
  // set and d0 is a RoPE dim; otherwise valid dummy addresses)
  const bool rot = a.nr_inv != nullptr && d0 >= a.d_nope;
  const f32x2 inv2 = *(const f32x2*)(rot ? a.nr_inv + ((d0 - a.d_nope) >> 1) : (const float*)a.pos);
  const int64_t p_row = a.pos[row];
  if (a.n_split <= kMergePhases * kMergeRegs) {
    // every split of this phase in registers before the first wait: the
    // maxima and the partials come in one round trip
    f32x2 mv[kMergeRegs];
    u32x2 ov[kMergeRegs];
#pragma unroll
    for (int i = 0; i < kMergeRegs; i++) {
      const int sp = ph + kMergePhases * i;
      mv[i] = (f32x2){-INFINITY, 0.f};
      ov[i] = (u32x2){0u, 0u};
      if (sp < a.n_split) {
        mv[i] = ml[(int64_t)sp * a.H];
        ov[i] = *(const u32x2*)(po + sp * sstride);
      }
    }
#pragma unroll
    for (int i = 0; i < kMergeRegs; i++) M = fmaxf(M, mv[i][0]);
    red[ph][vg][0] = M;
    __syncthreads();
    M = z2;
#pragma unroll
    for (int p = 0; p < kMergePhases; p++) M = fmaxf(M, red[p][vg][0]);
    if (M != -INFINITY) {
      // an empty split has m = -inf, hence weight 0, and zero partials
#pragma unroll
      for (int i = 0; i < kMergeRegs; i++) {
        if (ph + kMergePhases * i < a.n_split) {
          const float w = mv[i][1] * exp2f(mv[i][0] - M);
          den += w;
          acc[0] += w * bf16_bits_to_f32(ov[i][0] & 0xFFFFu);
          acc[1] += w * bf16_bits_to_f32(ov[i][0] >> 16);
          acc[2] += w * bf16_bits_to_f32(ov[i][1] & 0xFFFFu);
          acc[3] += w * bf16_bits_to_f32(ov[i][1] >> 16);
        }
      }
    }
  } else {
    // ---- the maximum over all splits (and the sink)
#pragma unroll 4
    for (int sp = ph; sp < a.n_split; sp += kMergePhases) M = fmaxf(M, ml[(int64_t)sp * a.H][0]);
    red[ph][vg][0] = M;
    __syncthreads();
    M = z2;
#pragma unroll
    for (int p = 0; p < kMergePhases; p++) M = fmaxf(M, red[p][vg][0]);
    // ---- this phase's weighted sums
    if (M != -INFINITY) {
#pragma unroll 4
      for (int sp = ph; sp < a.n_split; sp += kMergePhases) {
        const f32x2 v_ml = ml[(int64_t)sp * a.H];
        const u32x2 v = *(const u32x2*)(po + sp * sstride);
        const float w = v_ml[1] * exp2f(v_ml[0] - M);
        den += w;
        acc[0] += w * bf16_bits_to_f32(v[0] & 0xFFFFu);
        acc[1] += w * bf16_bits_to_f32(v[0] >> 16);
        acc[2] += w * bf16_bits_to_f32(v[1] & 0xFFFFu);
        acc[3] += w * bf16_bits_to_f32(v[1] >> 16);
      }
    }
  }
  red[ph][vg][1] = den;
#pragma unroll
  for (int i = 0; i < 4; i++) red[ph][vg][2 + i] = acc[i];
  __syncthreads();
  if (ph != 0 || !active) return;
  den = (M == -INFINITY || z2 == -INFINITY) ? 0.f : exp2f(z2 - M);
  float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < kMergePhases; p++) {
    den += red[p][vg][1];
#pragma unroll
    for (int i = 0; i < 4; i++) o[i] += red[p][vg][2 + i];
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  const int64_t oi = ((int64_t)row * a.H + head) * D + d0;
#pragma unroll
  for (int i = 0; i < 4; i++) o[i] *= inv;
  if (rot) {
    const float inv[2] = {inv2[0], inv2[1]};
    unrotate4(o, inv, 0, p_row);
  }
  if (a.out_bf16) {
    __builtin_nontemporal_store(pack4(o), (u32x2*)((uint16_t*)a.out + oi));
  } else {
    *(f32x4*)((float*)a.out + oi) = (f32x4){o[0], o[1], o[2], o[3]};
  }
}

// ---------------------------------------------------------------- plan / launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The split of the entry list depends only on the per-query bound on the
// number of entries, never on B or Q, so a sequence's result is the same at
// any batch size.
void attend_plan(AttendArgs& a, int64_t n_entries_max) {
  const int D = a.d_nope + a.d_rope;
  a.part_bf16 = a.fp8;
  a.f32_heads = a.fp8 ? 64 : (a.H < 4096 / D ? a.H : (4096 / D > 0 ? 4096 / D : 1));
  // short lists (CSA: k + window) split finer than long ones (HCA), so that
  // a small batch still spreads over the chip; the size depends on the
  // per-query bound only (short: ~17 splits of whole tiles, at least 64
  // entries -- 4-tile splits at top-2048 cost the B = 4 decode call 1 % and
  // save the 4096-query prefill 14 % of its CSA attention against 3-tile
  // splits; long: ~16 splits of whole tiles -- 544 entries for the
  // 8320-entry HCA list, 16 splits, so that B = 16 x 2 head groups fill
  // 512 workgroup slots, two per CU, in one round)
  int64_t per;
  if (n_entries_max <= 4096) {
    per = (n_entries_max + 16) / 17;
    if (per < 64) per = 64;
    per = (per + kTile - 1) / kTile * kTile;
  } else {
    per = (n_entries_max + 15) / 16;
    per = (per + kTile - 1) / kTile * kTile;
  }
  if (per > kMaxSplit) per = kMaxSplit;
  a.split_size = (int)per;
  int64_t ns = n_entries_max > 0 ? (n_entries_max + per - 1) / per : 1;
  a.n_split = (int)ns;
}

// partial O: bf16 on the FP8 path, fp32 on the fp32 path; the workspace
// query sizes for fp32 (the larger of the two)
static size_t part_elem(const AttendArgs& a) { return a.part_bf16 ? 2 : 4; }

size_t attend_workspace_bytes(const AttendArgs& a) {
  if (a.n_split <= 1) return 0;
  const size_t R = (size_t)a.B * a.Q, D = a.d_nope + a.d_rope;
  return align256(R * a.n_split * a.H * D * part_elem(a)) +
         align256(R * a.n_split * a.H * 2 * sizeof(float));
}

void attend_carve(AttendArgs& a, void* ws) {
  if (a.n_split <= 1) { a.part_o = nullptr; a.part_ml = nullptr; return; }
  const size_t R = (size_t)a.B * a.Q, D = a.d_nope + a.d_rope;
  a.part_o = ws;
  a.part_ml = (float*)((char*)ws + align256(R * a.n_split * a.H * D * part_elem(a)));
}

size_t attend_f32_smem(const AttendArgs& a) {
  const int D = a.d_nope + a.d_rope;
  return sizeof(float) * ((size_t)kF32Chunk * D + (size_t)a.f32_heads * D +
                          (size_t)a.f32_heads * kF32Chunk + 3 * (size_t)a.f32_heads) +
         sizeof(int) * kF32Chunk;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st, const KernelEvents* ev) {
  const int rows = a.B * a.Q;
  if (rows == 0) return hipSuccess;
  if (a.fp8) {
    const int64_t N = (int64_t)rows * a.n_split * ((a.H + kHeads - 1) / kHeads);
    const int64_t per = (N + 7) / 8;
    const bool nr = a.nr_gamma || a.nr_inv;
    // streaming loads for one-query CSA calls (decode: a query's gathered
    // rows are read by its two head groups only, and keeping them in L2
    // costs the calls that follow more than it saves: a 51.5 against
    // 54.1 us CSA layer); plain loads everywhere else (HCA rows are shared
    // by the head groups, a chunk's queries share rows: 44.6 against 46.9 us
    // HCA layer, and the prefill chunk 17.9 -> 16.0 ms).  The choice changes
    // no result.
    const bool stream = a.csa && a.Q == 1;
    const dim3 grid((unsigned)(8 * per)), block(kThreads);
    auto go = [&](auto kern) {
      if (ev)
        hipExtLaunchKernelGGL(kern, grid, block, 0, st, ev->start, ev->stop, 0, a);
      else
        hipLaunchKernelGGL(kern, grid, block, 0, st, a);
    };
    if (a.sel_ctr)
      stream ? go(k_attend_fp8_sel<true>) : go(k_attend_fp8_sel<false>);
    else if (nr)
      stream ? go(k_attend_fp8_nr<true>) : go(k_attend_fp8_nr<false>);
    else
      stream ? go(k_attend_fp8<true>) : go(k_attend_fp8<false>);
  } else {
    dim3 grid(rows, a.n_split, (a.H + a.f32_heads - 1) / a.f32_heads);
    if (ev)
      hipExtLaunchKernelGGL(k_attend_f32, grid, dim3(256), attend_f32_smem(a), st, ev->start,
                            ev->stop, 0, a);
    else
      hipLaunchKernelGGL(k_attend_f32, grid, dim3(256), attend_f32_smem(a), st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  if (a.fp8) {
    // 32 heads x 512 dims / (64 value groups x 4 values) = 64 workgroups per block
    const int parts = (kHeads * (kNope + kRope)) / (64 * 4);
    hipLaunchKernelGGL(k_merge_tiled, dim3(rows, (a.H + kHeads - 1) / kHeads, parts), dim3(256), 0,
                       st, a);
  } else {
    hipLaunchKernelGGL(k_merge, dim3(rows, (a.H + kMergeHeads - 1) / kMergeHeads), dim3(256), 0, st,
                       a);
  }
  return hipGetLastError();
}

}  // namespace v4a
