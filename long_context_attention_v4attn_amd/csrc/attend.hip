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
//   k_attend_fp8  gfx950 MFMA path.  A workgroup = 4 waves = 64 query heads of
//                 one query; wave w owns heads 16w..16w+15.  The entry list is
//                 walked in tiles of 32 entries staged (raw FP8 codes + BF16
//                 RoPE + fp32 scale) in LDS once per workgroup and read by all
//                 four waves:
//                   S^T = K Q^T  with v_mfma_f32_16x16x32_bf16, K rows read
//                         with ds_read_b64 and widened e4m3 -> bf16 exactly,
//                         Q^T held in registers for the whole kernel;
//                   O^T += V^T P^T, V^T fragments read straight from the
//                         row-major tile with ds_read_b64_tr_b8 (transpose
//                         load), P^T taken from the S^T accumulators.
//                 The per-entry FP8 scale multiplies the non-RoPE logit and
//                 the non-RoPE probability in fp32, so decoding adds no
//                 rounding.  Online softmax in base 2 with a lazily updated
//                 running max (rescale only when the max grows by > 8).
//   k_attend_f32  fp32 VALU path for unquantised entries (any D <= 512).
//   k_merge       combines split partials in fixed split order.
#include "common.hpp"
#include "kernels.hpp"

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
constexpr int kRowBytes = kNope + 2 * kRope; // 576 staged bytes per entry
constexpr int kRowStride = 592;              // padded LDS row (bank spread)
constexpr int kChunks = kRowBytes / 16;      // 36 x 16-byte chunks per entry
constexpr int kTileChunks = kTile * kChunks; // 1152
constexpr int kThreads = 256;
constexpr int kChunksPerThread = (kTileChunks + kThreads - 1) / kThreads;  // 5
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.0f;             // lazy max-rescale threshold (log2 units)

struct __align__(16) Fp8Tile {
  uint8_t rows[kTile * kRowStride];
  float scale[kTile];
  int valid[kTile];
};

// Widen 8 e4m3 codes (two dwords) to 8 bf16 (exact).
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i++) r[i] = (__bf16)v[i];
  return r;
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

__device__ __forceinline__ void stage_load(const AttendArgs& a, const RowEntries& r, int row,
                                           int b, int tile_e0, int e_end, u32x4* regs,
                                           float* sc_reg, int* valid_reg) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kChunksPerThread; j++) {
    int c = t + j * kThreads;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < kTileChunks) {
      int e = c / kChunks, part = c % kChunks;
      int ue = tile_e0 + e;
      if (ue < e_end) {
        bool is_win;
        int64_t src = entry_source(a, r, row, ue, &is_win);
        if (src >= 0) {
          const uint8_t* nope = is_win ? a.w_nope : a.c_nope;
          const uint16_t* rope = is_win ? a.w_rope : a.c_rope;
          int64_t cap = is_win ? a.w_cap : a.c_cap;
          int64_t rowi = (int64_t)b * cap + src;
          if (part < kNope / 16)
            v = *(const u32x4*)(nope + rowi * kNope + part * 16);
          else
            v = *(const u32x4*)((const uint8_t*)(rope + rowi * kRope) + (part - kNope / 16) * 16);
        }
      }
    }
    regs[j] = v;
  }
  if (t < kTile) {
    int ue = tile_e0 + t;
    float s = 0.0f;
    int ok = 0;
    if (ue < e_end) {
      bool is_win;
      int64_t src = entry_source(a, r, row, ue, &is_win);
      if (src >= 0) {
        const float* sc = is_win ? a.w_scale : a.c_scale;
        int64_t cap = is_win ? a.w_cap : a.c_cap;
        s = sc[(int64_t)b * cap + src];
        ok = 1;
      }
    }
    *sc_reg = s;
    *valid_reg = ok;
  }
}

__device__ __forceinline__ void stage_store(Fp8Tile* tl, const u32x4* regs, float sc, int ok) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kChunksPerThread; j++) {
    int c = t + j * kThreads;
    if (c < kTileChunks) {
      int e = c / kChunks, part = c % kChunks;
      *(u32x4*)(tl->rows + e * kRowStride + part * 16) = regs[j];
    }
  }
  if (t < kTile) {
    tl->scale[t] = sc;
    tl->valid[t] = ok;
  }
}

__global__ void __launch_bounds__(256, 1) k_attend_fp8(AttendArgs a) {
  __shared__ Fp8Tile tiles[2];
  const int row = blockIdx.x;              // b * Q + j
  const int split = blockIdx.y;
  const int hg = blockIdx.z;               // group of 64 heads
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = row / a.Q;
  const int g = lane >> 4;                 // lane group 0..3
  const int li = lane & 15;
  const int head = hg * 64 + wave * 16 + li;
  const bool head_ok = head < a.H;
  const int D = kNope + kRope;

  RowEntries r = row_entries(a, row);
  const int n_tot = r.n_c + r.n_w;
  const int e_beg = split * a.split_size;
  const int e_end = min(e_beg + a.split_size, n_tot);

  // Q^T fragments: k-step ks covers dims 32ks .. 32ks+31; lane holds dims
  // 32ks + 8g .. +8 of its head (zero for heads beyond H).
  bf16x8 qf[16];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)row * a.H + (head_ok ? head : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < 16; ks++) {
      u32x4 v = *(const u32x4*)(qp + ks * 32 + g * 8);
      if (!head_ok) v = (u32x4){0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 acc[32];                           // O^T blocks: 28 nope + 4 rope, 16 dims each
#pragma unroll
  for (int i = 0; i < 32; i++) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;                 // running max used for P (log2 units)
  float l_run = 0.0f;                      // lane-partial denominator
  const float c2 = a.sm_scale * kLog2e;

  const int n_tiles = e_end > e_beg ? (e_end - e_beg + kTile - 1) / kTile : 0;
  u32x4 regs[kChunksPerThread];
  float sc_reg = 0.f;
  int valid_reg = 0;
  if (n_tiles > 0) {
    stage_load(a, r, row, b, e_beg, e_end, regs, &sc_reg, &valid_reg);
    stage_store(&tiles[0], regs, sc_reg, valid_reg);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; it++) {
    const Fp8Tile* tl = &tiles[it & 1];
    const bool more = it + 1 < n_tiles;
    if (more) stage_load(a, r, row, b, e_beg + (it + 1) * kTile, e_end, regs, &sc_reg, &valid_reg);

    // ---- S^T = K Q^T for the two 16-entry row blocks
    f32x4 sn[2], sr[2];
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
      sn[rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
      sr[rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
      const uint8_t* kr = tl->rows + (rb * 16 + li) * kRowStride + g * 8;
#pragma unroll
      for (int ks = 0; ks < 14; ks++) {
        u32x2 w = *(const u32x2*)(kr + ks * 32);
        sn[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(w[0], w[1]), qf[ks], sn[rb], 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        u32x4 v = *(const u32x4*)(tl->rows + (rb * 16 + li) * kRowStride + kNope + ks * 64 + g * 16);
        sr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), qf[14 + ks],
                                                         sr[rb], 0, 0, 0);
      }
    }

    // ---- logits (log2 units), masked entries -> -inf
    float s2[8], scl[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int e = rb * 16 + g * 4 + i;
        float sc = tl->scale[e];
        bool ok = tl->valid[e] != 0;
        float v = (sn[rb][i] * sc + sr[rb][i]) * c2;
        v = ok ? v : -INFINITY;
        s2[rb * 4 + i] = v;
        scl[rb * 4 + i] = sc;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // lazy rescale: move the running max only when it grows by more than
    // kRescale (exact: P <= 2^kRescale and the final normalisation uses the
    // same max)
    bool need = (m_run == -INFINITY) ? (tmax > -INFINITY) : (tmax > m_run + kRescale);
    if (__builtin_amdgcn_ballot_w64(need)) {
      float m_new = need ? tmax : m_run;
      float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
      if (need) {
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 32; i++) acc[i] *= alpha;
        m_run = m_new;
      }
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    float pv[8], pn[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float p = exp2f(s2[i] - m_use);
      l_run += p;
      pv[i] = p;
      pn[i] = p * scl[i];
    }
    const bf16x8 pB = pack8(pv);           // P^T  (RoPE dims)
    const bf16x8 pnB = pack8(pn);          // (P * scale)^T (FP8 dims)

    // ---- O^T += V^T P^T; lane group g's k-values are entries
    // {4g..4g+3, 16+4g..16+4g+3}; source lane s of the group points at the
    // entry k = s/2 (tr8) resp. s/4 (tr16)
    {
      const int s = li;
      const int kk8 = s >> 1;
      const int ent8 = (kk8 < 4) ? (g * 4 + kk8) : (16 + g * 4 + kk8 - 4);
      const uint8_t* vb8 = tl->rows + ent8 * kRowStride + (s & 1) * 8;
#pragma unroll
      for (int db = 0; db < 28; db++) {
        u32x2 w = lds_tr8(vb8 + db * 16);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8(w[0], w[1]), pnB, acc[db], 0, 0, 0);
      }
      const int kk16 = s >> 2;
      const uint8_t* vlo = tl->rows + (g * 4 + kk16) * kRowStride + kNope + (s & 3) * 8;
      const uint8_t* vhi = tl->rows + (16 + g * 4 + kk16) * kRowStride + kNope + (s & 3) * 8;
#pragma unroll
      for (int db = 0; db < 4; db++) {
        u32x2 lo = lds_tr16(vlo + db * 32);
        u32x2 hi = lds_tr16(vhi + db * 32);
        u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
        acc[28 + db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pB,
                                                               acc[28 + db], 0, 0, 0);
      }
    }

    if (more) stage_store(&tiles[(it + 1) & 1], regs, sc_reg, valid_reg);
    __syncthreads();
  }

  // ---- epilogue: lane (g, li) holds O^T dims 16db + 4g + i of head `head`
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!head_ok) return;
  if (a.n_split == 1) {
    float z2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
    float M = fmaxf(m_run, z2);
    float so = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - M);
    float den = l_tot * so + ((z2 == -INFINITY) ? 0.0f : exp2f(z2 - M));
    float f = den > 0.0f ? so / den : 0.0f;
    int64_t ob = ((int64_t)row * a.H + head) * D;
#pragma unroll
    for (int db = 0; db < 32; db++) {
      int d0 = db * 16 + g * 4;
      f32x4 o = acc[db] * f;
      if (a.out_bf16) {
        uint32_t lo = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
        uint32_t hi = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
        *(u32x2*)((uint16_t*)a.out + ob + d0) = (u32x2){lo, hi};
      } else {
        *(f32x4*)((float*)a.out + ob + d0) = o;
      }
    }
  } else {
    int64_t pi = ((int64_t)row * a.n_split + split) * a.H + head;
#pragma unroll
    for (int db = 0; db < 32; db++) *(f32x4*)(a.part_o + pi * D + db * 16 + g * 4) = acc[db];
    if (g == 0) {
      a.part_ml[pi * 2 + 0] = m_run;
      a.part_ml[pi * 2 + 1] = l_tot;
    }
  }
}

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
      int64_t pi = ((int64_t)row * a.n_split + split) * a.H + head;
      a.part_o[pi * D + d] = o[j];
      if (d == 0) {
        a.part_ml[pi * 2] = mrun[h];
        a.part_ml[pi * 2 + 1] = lrun[h];
      }
    }
  }
}

// ---------------------------------------------------------------- merge
// out[row][h][:] = sum_s O_s 2^(m_s - M) / (sum_s l_s 2^(m_s - M) + 2^(z - M)),
// splits visited in index order (deterministic).
__global__ void __launch_bounds__(256) k_merge(AttendArgs a) {
  const int row = blockIdx.x;
  const int head = blockIdx.y;
  const int D = a.d_nope + a.d_rope;
  const float* ml = a.part_ml + ((int64_t)row * a.n_split * a.H) * 2;
  float z2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
  float M = z2;
  for (int s = 0; s < a.n_split; s++) M = fmaxf(M, ml[((int64_t)s * a.H + head) * 2]);
  float den = (z2 == -INFINITY || M == -INFINITY) ? 0.f : exp2f(z2 - M);
  for (int s = 0; s < a.n_split; s++) {
    float m = ml[((int64_t)s * a.H + head) * 2];
    if (m != -INFINITY) den += ml[((int64_t)s * a.H + head) * 2 + 1] * exp2f(m - M);
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < a.n_split; s++) {
      float m = ml[((int64_t)s * a.H + head) * 2];
      if (m == -INFINITY) continue;
      acc += a.part_o[(((int64_t)row * a.n_split + s) * a.H + head) * D + d] * exp2f(m - M);
    }
    float v = acc * inv;
    int64_t oi = ((int64_t)row * a.H + head) * D + d;
    if (a.out_bf16) ((uint16_t*)a.out)[oi] = (uint16_t)f32_to_bf16_bits(v);
    else ((float*)a.out)[oi] = v;
  }
}

// ---------------------------------------------------------------- plan / launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The split of the entry list depends only on the per-query bound on the
// number of entries, never on B or Q, so a sequence's result is the same at
// any batch size.
void attend_plan(AttendArgs& a, int64_t n_entries_max) {
  const int D = a.d_nope + a.d_rope;
  a.f32_heads = a.fp8 ? 64 : (a.H < 4096 / D ? a.H : (4096 / D > 0 ? 4096 / D : 1));
  int64_t per = (n_entries_max + 15) / 16;
  if (per < 128) per = 128;
  per = (per + 31) / 32 * 32;
  a.split_size = (int)per;
  int64_t ns = n_entries_max > 0 ? (n_entries_max + per - 1) / per : 1;
  a.n_split = (int)ns;
}

size_t attend_workspace_bytes(const AttendArgs& a) {
  if (a.n_split <= 1) return 0;
  const size_t R = (size_t)a.B * a.Q, D = a.d_nope + a.d_rope;
  return align256(R * a.n_split * a.H * D * sizeof(float)) +
         align256(R * a.n_split * a.H * 2 * sizeof(float));
}

void attend_carve(AttendArgs& a, void* ws) {
  if (a.n_split <= 1) { a.part_o = nullptr; a.part_ml = nullptr; return; }
  const size_t R = (size_t)a.B * a.Q, D = a.d_nope + a.d_rope;
  a.part_o = (float*)ws;
  a.part_ml = (float*)((char*)ws + align256(R * a.n_split * a.H * D * sizeof(float)));
}

size_t attend_f32_smem(const AttendArgs& a) {
  const int D = a.d_nope + a.d_rope;
  return sizeof(float) * ((size_t)kF32Chunk * D + (size_t)a.f32_heads * D +
                          (size_t)a.f32_heads * kF32Chunk + 3 * (size_t)a.f32_heads) +
         sizeof(int) * kF32Chunk;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  const int rows = a.B * a.Q;
  if (rows == 0) return hipSuccess;
  if (a.fp8) {
    dim3 grid(rows, a.n_split, (a.H + 63) / 64);
    hipLaunchKernelGGL(k_attend_fp8, grid, dim3(kThreads), 0, st, a);
  } else {
    dim3 grid(rows, a.n_split, (a.H + a.f32_heads - 1) / a.f32_heads);
    hipLaunchKernelGGL(k_attend_f32, grid, dim3(256), attend_f32_smem(a), st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  hipLaunchKernelGGL(k_merge, dim3(rows, a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace v4a
