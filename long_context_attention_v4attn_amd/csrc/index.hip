// Lightning indexer and top-k selector.
//
// Method: [Notes §7] index score I_{t,s} = sum_h w_{t,h} ReLU(q_{t,h} . K_s)
// over the compressed blocks visible to query t, then Top-k over s;
// [Notes §9] the indexer's QK path runs in FP4 (keys and queries MXFP4), and
// the selector ranks fp32 scores.
//
// Kernels
//   k_quant_q     query heads -> MXFP4 (e2m1 codes + e8m0 scale per 32).
//   k_score_mx    FP4 scan: one v_mfma_scale_f32_16x16x128_f8f6f4 per
//                 (16 heads, 16 blocks); M = index heads, N = blocks, K = 128
//                 dims; the e8m0 block scales feed the MFMA's scale operands,
//                 so products are exact.  The ReLU / head-weight sum is an
//                 fp32 epilogue: in-lane over 4 heads, then across the four
//                 lane groups.  Keys stream in coalesced 1 KB wave loads.
//   k_score_f32   fp32 VALU dot products for unquantised keys.
//   k_select      exact top-k per query: radix select on the 64-bit key
//                 (order-preserving fp32 score bits, inverted block id) in
//                 11/11/10-bit digits with LDS histograms; stops as soon as
//                 the threshold bin holds exactly the remaining count; the
//                 selected ids are then compacted in ascending order with a
//                 block scan (so the output is deterministic), -1 padded.
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t index_workspace_bytes(int B, int Q, int H, int d, int64_t cap, int key_mx) {
  const size_t R = (size_t)B * Q;
  size_t n = 0;
  if (key_mx) n += align256(R * H * (d / 2)) + align256(R * H * (d / 32));
  n += align256(R * (size_t)cap * sizeof(float));
  return n;
}

void index_carve(IndexArgs& a, void* ws) {
  const size_t R = (size_t)a.B * a.Q;
  char* p = (char*)ws;
  if (a.key_mx) {
    a.qmx = (uint8_t*)p;
    p += align256(R * a.H * (a.d / 2));
    a.qsc = (uint8_t*)p;
    p += align256(R * a.H * (a.d / 32));
  } else {
    a.qmx = nullptr;
    a.qsc = nullptr;
  }
  a.scores = (float*)p;
}

__device__ __forceinline__ int64_t n_visible(int64_t p, int m, int64_t cap) {
  if (p < 0) return 0;
  int64_t nv = (p + 1) / m;
  return nv < cap ? nv : cap;
}

// ---------------------------------------------------------------- query MXFP4
// One wave per (row, head): 128 elements, 2 per lane; a group of 32 elements
// is 16 lanes.
__global__ void __launch_bounds__(256) k_quant_q(IndexArgs a) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const int R = a.B * a.Q;
  if (wave >= R * a.H) return;
  const size_t base = (size_t)wave * a.d;
  float x0 = load_as_f32(a.q, a.q_bf16, base + 2 * lane);
  float x1 = load_as_f32(a.q, a.q_bf16, base + 2 * lane + 1);
  float am = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  int e = mx_exponent(am);
  float inv = ldexpf(1.0f, -e);
  uint32_t c0 = am > 0.f ? enc_e2m1(x0 * inv) : 0u;
  uint32_t c1 = am > 0.f ? enc_e2m1(x1 * inv) : 0u;
  a.qmx[(size_t)wave * (a.d / 2) + lane] = (uint8_t)(c0 | (c1 << 4));
  if ((lane & 15) == 0) a.qsc[(size_t)wave * (a.d / 32) + (lane >> 4)] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------- FP4 scan
// Workgroup = 4 waves x 64 blocks = 256 consecutive blocks of one query.
constexpr int kScoreBlocks = 256;

__global__ void __launch_bounds__(256) k_score_mx(IndexArgs a) {
  const int row = blockIdx.y;
  const int b = row / a.Q;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int64_t blk0 = (int64_t)blockIdx.x * kScoreBlocks + wave * 64;
  if (blk0 >= nv) return;
  const int HT = a.H / 16;

  // A operands: q heads (ht*16 + li), 32 elements of group g
  i32x8 qa[4];
  int qs[4];
  float wv[4][4];
  for (int ht = 0; ht < HT; ht++) {
    const uint8_t* qp = a.qmx + ((size_t)row * a.H + ht * 16 + li) * 64 + g * 16;
    u32x4 v = *(const u32x4*)qp;
    qa[ht] = (i32x8){(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
    qs[ht] = a.qsc[((size_t)row * a.H + ht * 16 + li) * 4 + g];
#pragma unroll
    for (int i = 0; i < 4; i++) wv[ht][i] = a.w[(size_t)row * a.H + ht * 16 + g * 4 + i];
  }
  const uint8_t* kc = (const uint8_t*)a.codes + (size_t)b * a.cap * 64;
  const uint8_t* ks = a.kscales + (size_t)b * a.cap * 4;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int64_t blk = blk0 + t * 16 + li;
    const bool ok = blk < nv;
    u32x4 v = {0u, 0u, 0u, 0u};
    int sc = 127;
    if (ok) {
      v = *(const u32x4*)(kc + blk * 64 + g * 16);
      sc = ks[blk * 4 + g];
    }
    i32x8 kb = {(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
    float part = 0.0f;
    for (int ht = 0; ht < HT; ht++) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht], kb, acc, 4, 4, 0, qs[ht], 0, sc);
#pragma unroll
      for (int i = 0; i < 4; i++) part += wv[ht][i] * fmaxf(acc[i], 0.0f);
    }
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if (g == 0 && ok) a.scores[(size_t)row * a.cap + blk] = part;
  }
}

// ---------------------------------------------------------------- fp32 scan
__global__ void __launch_bounds__(256) k_score_f32(IndexArgs a) {
  extern __shared__ float qsm[];          // [H][d] then w[H]
  const int row = blockIdx.y;
  const int b = row / a.Q;
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  float* wsm = qsm + a.H * a.d;
  for (int i = threadIdx.x; i < a.H * a.d; i += blockDim.x)
    qsm[i] = load_as_f32(a.q, a.q_bf16, (size_t)row * a.H * a.d + i);
  for (int i = threadIdx.x; i < a.H; i += blockDim.x) wsm[i] = a.w[(size_t)row * a.H + i];
  __syncthreads();
  if (blk >= nv) return;
  const float* kr = (const float*)a.codes + ((size_t)b * a.cap + blk) * a.d;
  float s = 0.0f;
  for (int h = 0; h < a.H; h++) {
    float dot = 0.0f;
    for (int c = 0; c < a.d; c++) dot += qsm[h * a.d + c] * kr[c];
    s += wsm[h] * fmaxf(dot, 0.0f);
  }
  a.scores[(size_t)row * a.cap + blk] = s;
}

// ---------------------------------------------------------------- select
constexpr int kSelThreads = 512;
constexpr int kBins = 2048;

// Inclusive block scan of one value per thread (kSelThreads threads).
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w = 0; w < wave; w++) add += tmp[w];
  __syncthreads();
  return v + add;
}

// 64-bit selection key of element i: higher = better (score desc, id asc).
__device__ __forceinline__ uint64_t sel_key(const float* sc, int64_t i) {
  float f = sc[i];
  if (f == 0.0f) f = 0.0f;                 // -0 ranks equal to +0
  return ((uint64_t)order_key(f) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

__global__ void __launch_bounds__(kSelThreads) k_select(IndexArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t tmp[kSelThreads / 64];
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ uint32_t s_need, s_tot;
  __shared__ int s_done;
  const int row = blockIdx.x;
  const int64_t nv = n_visible(a.pos[row], a.m, a.cap);
  const int k = a.k;
  const int64_t kk = nv < k ? nv : k;
  const float* sc = a.scores + (size_t)row * a.cap;
  int32_t* out = a.topk + (size_t)row * k;

  if (kk == nv) {                          // everything visible is selected
    for (int64_t i = threadIdx.x; i < k; i += blockDim.x) out[i] = i < nv ? (int32_t)i : -1;
    return;
  }
  if (threadIdx.x == 0) {
    s_prefix = 0;
    s_mask = 0;
    s_need = (uint32_t)kk;
    s_done = 0;
  }
  __syncthreads();

  // digits (shift, width) over the 64-bit key, most significant first
  const int shifts[6] = {53, 42, 32, 21, 10, 0};
  const int widths[6] = {11, 11, 10, 11, 11, 10};
  for (int pass = 0; pass < 6; pass++) {
    if (s_done) break;
    const int sh = shifts[pass], wd = widths[pass];
    const uint32_t nb = 1u << wd;
    for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const uint64_t pm = s_mask, pp = s_prefix;
    for (int64_t i = threadIdx.x; i < nv; i += blockDim.x) {
      uint64_t key = sel_key(sc, i);
      if ((key & pm) == pp) atomicAdd(&hist[(uint32_t)(key >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    // suffix counts from the top bin: thread t owns bins nb-1-4t .. nb-4-4t
    const int per = (int)(nb + kSelThreads - 1) / kSelThreads;   // 4 or 2
    uint32_t cnt = 0;
    for (int j = 0; j < per; j++) {
      int bin = (int)nb - 1 - (threadIdx.x * per + j);
      if (bin >= 0) cnt += hist[bin];
    }
    uint32_t incl = block_incl_scan(cnt, tmp);
    uint32_t excl = incl - cnt;
    const uint32_t need = s_need;
    if (excl < need && incl >= need) {     // exactly one thread
      uint32_t above = excl;
      for (int j = 0; j < per; j++) {
        int bin = (int)nb - 1 - (threadIdx.x * per + j);
        uint32_t h = hist[bin];
        if (above + h >= need) {
          uint32_t rem = need - above;
          s_prefix = pp | ((uint64_t)bin << sh);
          s_mask = pm | ((uint64_t)(nb - 1) << sh);
          s_need = rem;
          if (h == rem) s_done = 1;
          break;
        }
        above += h;
      }
    }
    __syncthreads();
  }
  // a fully resolved 64-bit key is unique, so (key & mask) >= prefix selects
  // exactly kk elements; compact them in ascending id order
  const uint64_t pm = s_mask, pp = s_prefix;
  uint32_t base = 0;
  for (int64_t c0 = 0; c0 < nv; c0 += blockDim.x) {
    int64_t i = c0 + threadIdx.x;
    uint32_t f = (i < nv && (sel_key(sc, i) & pm) >= pp) ? 1u : 0u;
    uint32_t incl = block_incl_scan(f, tmp);
    if (f && base + incl - 1 < (uint32_t)kk) out[base + incl - 1] = (int32_t)i;
    if (threadIdx.x == blockDim.x - 1) s_tot = incl;
    __syncthreads();
    base += s_tot;
    __syncthreads();
  }
  for (int64_t i = kk + threadIdx.x; i < k; i += blockDim.x) out[i] = -1;
}

hipError_t launch_index_topk(const IndexArgs& a, hipStream_t st) {
  const int R = a.B * a.Q;
  if (R == 0) return hipSuccess;
  if (a.key_mx) {
    const int waves = R * a.H;
    hipLaunchKernelGGL(k_quant_q, dim3((waves + 3) / 4), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)((a.cap + kScoreBlocks - 1) / kScoreBlocks), R);
    hipLaunchKernelGGL(k_score_mx, grid, dim3(256), 0, st, a);
  } else {
    dim3 grid((unsigned)((a.cap + 255) / 256), R);
    size_t smem = sizeof(float) * ((size_t)a.H * a.d + a.H);
    hipLaunchKernelGGL(k_score_f32, grid, dim3(256), smem, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select, dim3(R), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace v4a
