// Top-k selection primitives shared by the selector kernels and the CSA
// attention's fused prologue: the order-preserving score keys, the 64-bit
// selection key (score key : inverted id), the filters' chunking and
// counters, block scans, the histogram bin search and the exact threshold
// resolution among the candidates ([Notes §7] Top-k; ties go to the lower id).
#pragma once

#include "common.hpp"

namespace v4a {

constexpr int kBins1 = 256;                // first radix digit: key bits 31..24
constexpr int kSh1 = 24;
constexpr int kBins2 = 2048;               // second digit: key bits 23..13
constexpr int kSh2 = 13;
constexpr int kBinsMax = 4096;             // widest digit of the final select
constexpr int kCandCap = 16384;            // candidate slots per query
constexpr int kFThreads = 256;
constexpr int kPer = 16;                   // consecutive scores per filter thread
constexpr int kFilterChunk = kFThreads * kPer;   // scores per filter workgroup
static_assert(kBins1 == kFThreads, "one first-digit bin per filter thread");
constexpr int kCtr = 8;                    // counters per query
constexpr int kFbSlot = 1;                 // counter slot: the row takes the full-score path
constexpr int kCntSlot = 6;                // counter slot: candidates above the sampled threshold
constexpr int kThrSlot = 7;                // counter slot: the sampled threshold key
__host__ __device__ inline int64_t score_ld(int64_t cap) { return (cap + 63) / 64 * 64; }
__host__ __device__ inline int64_t n_chunks(int64_t cap) { return (cap + kFilterChunk - 1) / kFilterChunk; }

__device__ __forceinline__ int64_t n_visible(int64_t p, int m, int64_t cap) {
  if (p < 0) return 0;
  int64_t nv = (p + 1) / m;
  return nv < cap ? nv : cap;
}

// Order-preserving key of a score; -0 is ranked equal to +0.
__device__ __forceinline__ uint32_t score_key(float f) {
  if (f == 0.0f) f = 0.0f;
  return order_key(f);
}

// The 64-bit selection key of id i: score key above, inverted id below, so
// that of two equal scores the lower id ranks higher.
__device__ __forceinline__ uint64_t sel_key(uint32_t k32, int64_t i) {
  return ((uint64_t)k32 << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

// Inclusive scan over the 64 lanes of a wave with DPP moves (no LDS round
// trips): row_shr 1, 2, 4, 8 scan each row of 16 lanes, then row_bcast15
// adds row 0's total to row 1 and row 2's to row 3, and row_bcast31 adds
// lane 31's (rows 0-1) to rows 2 and 3.  A lane whose source lies outside
// its row, or whose row is masked off, receives the old value 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// Inclusive block scan of one value per thread.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* tmp,
                                                    uint32_t* total = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  uint32_t add = 0, all = 0;
  for (int w = 0; w < kFThreads / 64; w++) {
    add += w < wave ? tmp[w] : 0u;
    all += tmp[w];
  }
  if (total) *total = all;
  __syncthreads();
  return v + add;
}

// Find the bin (scanning from the top) where the cumulative count reaches
// `need` (1 <= need <= total); writes (bin, count strictly above) to shared
// memory.  All threads must call it; nb is a power of two (a multiple of
// kFThreads, or below it: one bin per thread, the rest empty).
static __device__ void find_bin(const uint32_t* h, int nb, uint32_t need, uint32_t* tmp,
                                int* s_bin, uint32_t* s_above) {
  const int per = nb >= kFThreads ? nb / kFThreads : 1;
  uint32_t cnt = 0;
  for (int j = 0; j < per; j++) {
    const int i = threadIdx.x * per + j;
    cnt += i < nb ? h[nb - 1 - i] : 0u;
  }
  uint32_t incl = block_incl_scan(cnt, tmp);
  uint32_t excl = incl - cnt;
  if (excl < need && incl >= need) {
    uint32_t above = excl;
    for (int j = 0; j < per; j++) {
      int bin = nb - 1 - (threadIdx.x * per + j);      // >= 0: this thread's count is not empty
      if (above + h[bin] >= need) {
        *s_bin = bin;
        *s_above = above;
        break;
      }
      above += h[bin];
    }
  }
  __syncthreads();
}

// Candidates of the threshold search: the compact list (in LDS, or the
// query's global list), or (when it overflowed) the query's scores filtered
// by the candidates' common key prefix (the top pbits bits of the score key;
// pbits = 0: no common prefix).
struct CandSrc {
  const uint64_t* lds;                     // the list in LDS, or null
  const uint64_t* glob;                    // the query's global list
  uint32_t n;
  const float* sc;                         // the query's score row
  int64_t nv;
  uint32_t pfx;
  int pbits;
  bool compact;
  __device__ __forceinline__ int64_t size() const { return compact ? (int64_t)n : nv; }
  __device__ __forceinline__ bool get(int64_t i, uint64_t* key) const {
    if (compact) {
      *key = lds ? lds[i] : glob[i];
      return true;
    }
    const uint32_t k32 = score_key(sc[i]);
    *key = sel_key(k32, i);
    return pbits == 0 || (k32 >> (32 - pbits)) == pfx;
  }
};

// Sum of one value per thread over the workgroup.
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* tmp) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int w = 0; w < kFThreads / 64; w++) t += tmp[w];
  __syncthreads();
  return t;
}

// The exact 64-bit threshold T: the need-th largest key among the
// candidates (radix select on the bits below the candidates' common key
// prefix).  Exactly `need` candidates have keys >= T.
static __device__ uint64_t resolve_threshold(const CandSrc& src, uint32_t need, uint32_t* lh,
                                             uint32_t* tmp) {
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ uint32_t s_need, s_above;
  __shared__ int s_bin, s_done;
  if (threadIdx.x == 0) {
    s_prefix = src.pbits ? (uint64_t)src.pfx << (64 - src.pbits) : 0ull;
    s_mask = src.pbits ? (((uint64_t)1 << src.pbits) - 1) << (64 - src.pbits) : 0ull;
    s_need = need;
    s_done = 0;
  }
  __syncthreads();
  // remaining digits: the score key bits below the prefix, then the
  // inverted id, 11 bits a pass from the top (all that is left once 12 or
  // fewer remain)
  const int64_t n = src.size();
  for (int lo = 64 - src.pbits; lo > 0;) {
    if (s_done) break;
    const int wd = lo > 12 ? 11 : lo;
    const int sh = lo - wd;
    lo = sh;
    const uint32_t nb = 1u << wd;
    for (int i = threadIdx.x; i < (int)nb; i += blockDim.x) lh[i] = 0u;
    __syncthreads();
    const uint64_t pm = s_mask, pp = s_prefix;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
      uint64_t key;
      if (src.get(i, &key) && (key & pm) == pp) atomicAdd(&lh[(uint32_t)(key >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin(lh, (int)nb, s_need, tmp, &s_bin, &s_above);
    if (threadIdx.x == 0) {
      const uint32_t rem = s_need - s_above;
      s_prefix = pp | ((uint64_t)s_bin << sh);
      s_mask = pm | ((uint64_t)(nb - 1) << sh);
      // the whole bin is taken: the prefix with the remaining bits zero is
      // a threshold every key of the bin meets
      if (lh[s_bin] == rem) s_done = 1;
      s_need = rem;
    }
    __syncthreads();
  }
  const uint64_t T = s_prefix;
  __syncthreads();
  return T;
}

constexpr int kEmitCand = 4096;            // candidates resolved from LDS
constexpr int kRankCand = 128;             // candidates resolved by counting ranks

// The threshold when the candidates are few and in LDS: the keys are all
// distinct (the low word is the inverted id), so the need-th largest is the
// one candidate that exactly need - 1 others exceed.
static __device__ uint64_t rank_threshold(const uint64_t* cl, uint32_t n, uint32_t need) {
  __shared__ uint64_t s_T;
  if (threadIdx.x < n) {
    const uint64_t c = cl[threadIdx.x];
    uint32_t r = 0;
    for (uint32_t j = 0; j < n; j++) r += cl[j] > c ? 1u : 0u;
    if (r == need - 1) s_T = c;
  }
  __syncthreads();
  return s_T;
}

}  // namespace v4a
