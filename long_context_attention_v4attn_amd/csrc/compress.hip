// Token-level KV compressor: softmax-gated pooling with a learned positional
// bias, written straight into the cache format.
//
// Method: [Notes §8] HCA compressor S = Softmax_row(Z_block + B),
// C^Comp_i = sum_j S_j (elementwise) C_j over the m' tokens of block i (per
// channel, softmax across the block's rows); [Notes §7] CSA pools 2m adjacent
// entries from two streams with overlap; [HF "Hybrid attention"] softmax-gated
// pooling with a learned positional bias.  Overlap pairing used here: entry i
// pools the m previous-role rows of block i-1 and the m current-role rows of
// block i under one softmax (block 0: current rows only).
//
// k_compress: one workgroup per (block, sequence).  Each thread owns channels
// c = tid, tid + 256, ... and runs an online softmax over the block's slots
// (coalesced: adjacent threads read adjacent channels of the same token), in
// fp32.  The epilogue quantises the pooled row:
//   FP8 entry: workgroup max over the d_nope channels -> s = amax/448
//              (correctly rounded), e4m3 = RNE(clamp(y/s)); RoPE tail -> bf16.
//   MXFP4 key: 32 consecutive channels = 32 consecutive lanes; lane-shuffle
//              max -> e8m0 exponent, e2m1 = RNE(y * 2^-e); two nibbles a byte.
// k_append: a decode step ([Notes §11] state cache), one workgroup per
//   sequence.  The state holds, per channel, the running online-softmax
//   triple (max, denominator, numerator) of the block being pooled and of the
//   previous-role part of the next block, so a step folds in one token's rows
//   and a block completes with one divide: O(1) work per step, and the same
//   sequence of operations as k_compress (previous-role slots in order, then
//   current ones), hence the same values.
// k_append_batch: several appends (up to 8, each its own argument block) in
//   one launch, workgroup (b, j) = sequence b of append j.
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

constexpr int kCompThreads = 256;
constexpr int kMaxChan = 4;                // d <= 1024

__device__ __forceinline__ float ld(const void* p, int bf16, size_t i) {
  return load_as_f32(p, bf16, i);
}

// The input dtype as a template parameter: no branch around the load.
template <bool kBf16>
__device__ __forceinline__ float ldt(const void* p, size_t i) {
  if (kBf16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

// Stands in for an absent gate, bias or state row (zeros; any dtype, d <= 1024).
__device__ float g_zero_row[kMaxChan * kCompThreads];

// Online softmax step: fold slot (logit z, value v) into (mx, den, num).
// Branch-free; exp(0) = 1 exactly, so this is the same arithmetic as
// rescaling only when the maximum moves.
struct Acc {
  float mx, den, num;
};
__device__ __forceinline__ void acc_add(Acc& s, float z, float v) {
  const float mn = fmaxf(s.mx, z);
  const float sc = expf(s.mx - mn);        // mx = -inf -> 0
  const float e = expf(z - mn);
  s.den = s.den * sc + e;
  s.num = s.num * sc + e * v;
  s.mx = mn;
}

// Epilogue shared by the kernels: the pooled row y (channels tid + NT q) of
// block gblk of sequence b -> optional entry RMSNorm / RoPE -> the cache
// format, at the block's ring row or pool row.  Every thread of the
// workgroup calls it (it synchronises).
template <int NT>
__device__ __forceinline__ void finish_entry(const CompressArgs& a, float (&y)[1024 / NT], int b,
                                             int64_t gblk, float* red) {
  constexpr int kCh = 1024 / NT;           // channels per thread (d <= 1024)
  const int m = a.m;
  const int d = a.d;
  const int64_t orow = a.pg.tab ? page_row(a.pg, b, gblk) : (int64_t)b * a.cap + (gblk % a.cap);
  if (a.out_kind == 0 && (a.nr_gamma || a.nr_inv)) {
    // [Notes §9] KV-entry RMSNorm over the d channels, then RoPE of the last
    // d - d_nope channels at the entry's position (its block's last token):
    // adjacent channels pair up, and since d_nope and 256 are even a pair is
    // two adjacent lanes of one wave
    if (a.nr_gamma) {
      float ss = 0.0f;
#pragma unroll
      for (int q = 0; q < kCh; q++) ss += y[q] * y[q];   // y = 0 past d
      ss = wave_sum(ss);
      __syncthreads();                     // red is free
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
      __syncthreads();
      ss = red[0];
      for (int w = 1; w < NT / 64; w++) ss += red[w];
      __syncthreads();                     // red is reused below
      const float r = 1.0f / sqrtf(ss / (float)d + a.nr_eps);
#pragma unroll
      for (int q = 0; q < kCh; q++) {
        const int c = threadIdx.x + q * NT;
        if (c < d) y[q] = y[q] * r * a.nr_gamma[c];
      }
    }
    if (a.nr_inv) {
      const float pf = (float)(gblk * m + m - 1);
#pragma unroll
      for (int q = 0; q < kCh; q++) {
        const int c = threadIdx.x + q * NT;
        const float other = __shfl_xor(y[q], 1, 64);       // channel c ^ 1
        if (c < d && c >= a.d_nope) {
          const float ang = pf * a.nr_inv[(c - a.d_nope) >> 1];
          float sn, cs;
          sincos_angle(ang, &sn, &cs);
          y[q] = ((c - a.d_nope) & 1) ? other * sn + y[q] * cs : y[q] * cs - other * sn;
        }
      }
    }
  }
  if (a.out_kind == 0) {
    const int dn = a.d_nope, dr = d - a.d_nope;
    if (a.out_fmt == 0) {
#pragma unroll
      for (int q = 0; q < kCh; q++) {
        const int c = threadIdx.x + q * NT;
        if (c >= d) continue;
        if (c < dn) ((float*)a.o_a)[orow * dn + c] = y[q];
        else ((float*)a.o_b)[orow * dr + (c - dn)] = y[q];
      }
      return;
    }
    // FP8 entry: amax over the non-RoPE channels
    float am = 0.0f;
#pragma unroll
    for (int q = 0; q < kCh; q++) {
      const int c = threadIdx.x + q * NT;
      if (c < dn) am = fmaxf(am, fabsf(y[q]));
    }
    am = wave_max(am);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    am = red[0];
    for (int w = 1; w < NT / 64; w++) am = fmaxf(am, red[w]);
    const float s = am > 0.0f ? __fdiv_rn(am, kE4M3Max) : 1.0f;
#pragma unroll
    for (int q = 0; q < kCh; q++) {
      const int c = threadIdx.x + q * NT;
      if (c >= d) continue;
      if (c < dn) {
        float u = __fdiv_rn(y[q], s);
        u = fminf(fmaxf(u, -kE4M3Max), kE4M3Max);
        ((uint8_t*)a.o_a)[orow * dn + c] = (uint8_t)enc_e4m3(u);
      } else {
        ((uint16_t*)a.o_b)[orow * dr + (c - dn)] = (uint16_t)f32_to_bf16_bits(y[q]);
      }
    }
    if (threadIdx.x == 0) a.o_scale[orow] = s;
    return;
  }
  // indexer keys
  if (a.out_fmt == 0) {
#pragma unroll
    for (int q = 0; q < kCh; q++) {
      const int c = threadIdx.x + q * NT;
      if (c < d) ((float*)a.o_a)[orow * d + c] = y[q];
    }
    return;
  }
  // MXFP4: d % 32 == 0, so a group of 32 channels is 32 consecutive lanes
#pragma unroll
  for (int q = 0; q < kCh; q++) {
    const int c = threadIdx.x + q * NT;
    float v = c < d ? y[q] : 0.0f;
    float am = fabsf(v);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    const int e = mx_exponent(am);
    uint32_t code = am > 0.0f ? enc_e2m1(v * ldexpf(1.0f, -e)) : 0u;
    uint32_t hi = __shfl_down(code, 1, 64);
    if (c < d) {
      if ((c & 1) == 0) ((uint8_t*)a.o_a)[orow * (d / 2) + c / 2] = (uint8_t)(code | (hi << 4));
      if ((c & 31) == 0) ((uint8_t*)a.o_b)[orow * (d / 32) + c / 32] = (uint8_t)(e + 127);
    }
  }
}

__global__ void __launch_bounds__(kCompThreads) k_compress(CompressArgs a) {
  __shared__ float red[kCompThreads / 64];
  const int j = blockIdx.x;                // block within the call
  const int b = blockIdx.y;
  const int m = a.m;
  const int d = a.d;
  const bool overlap = a.kv_prev != nullptr;
  const int64_t gblk = a.t0 / m + j;       // global block index
  // a call that produces more than cap ring entries keeps the last cap of
  // them: an earlier block whose ring row a later block of this call also
  // writes is skipped (concurrent writes to one row would race)
  if (!a.pg.tab && (int64_t)(a.T / m) - j > a.cap) return;
  const bool has_prev = overlap && gblk > 0;
  const int64_t rbase = ((int64_t)b * a.T + (int64_t)j * m) * d;   // row m*j of this call

  float y[kMaxChan];
#pragma unroll
  for (int q = 0; q < kMaxChan; q++) {
    const int c = threadIdx.x + q * kCompThreads;
    y[q] = 0.0f;
    if (c >= d) continue;
    Acc s{-INFINITY, 0.0f, 0.0f};
    if (has_prev) {
      for (int u = 0; u < m; u++) {
        size_t idx = rbase + (int64_t)u * d + c;
        float z = (a.gate_prev ? ld(a.gate_prev, a.in_bf16, idx) : 0.0f) +
                  (a.bias ? a.bias[(size_t)u * d + c] : 0.0f);
        acc_add(s, z, ld(a.kv_prev, a.in_bf16, idx));
      }
    }
    const int boff = overlap ? m : 0;
    for (int u = 0; u < m; u++) {
      size_t idx = rbase + (int64_t)u * d + c;
      float z = (a.gate_cur ? ld(a.gate_cur, a.in_bf16, idx) : 0.0f) +
                (a.bias ? a.bias[(size_t)(boff + u) * d + c] : 0.0f);
      acc_add(s, z, ld(a.kv_cur, a.in_bf16, idx));
    }
    y[q] = s.num / s.den;
  }
  finish_entry<kCompThreads>(a, y, b, gblk, red);
}

// Large blocks (HCA, m' = 128 slots): one workgroup of kWideThreads per
// (block, sequence) with the slots spread over it.  A lane moves 16 bytes of
// a token row (VW channels); the d / VW lanes of a slot group cover the row,
// and the kWideThreads / (d / VW) groups take consecutive slot ranges (in
// slot order, eight slots' loads in flight per lane).  A chunk of eight
// slots is folded at once: the running max moves once per chunk and each
// slot costs one base-2 exponential (v_exp_f32).  Each group's
// (max, denominator, numerator) per channel goes to LDS and the groups are
// combined in group order (deterministic), then the shared epilogue.
constexpr int kWideThreads = 512;
constexpr int kWideUnroll = 8;
constexpr float kLog2eC = 1.4426950408889634f;

// (mx, den, num) of a later slot range folded into an earlier one.
__device__ __forceinline__ void acc_merge(Acc& r, const Acc& o) {
  if (o.mx == -INFINITY) return;           // an empty range
  if (r.mx == -INFINITY) {
    r = o;
    return;
  }
  const float mn = fmaxf(r.mx, o.mx);
  const float sa = expf(r.mx - mn), sb = expf(o.mx - mn);
  r.den = r.den * sa + o.den * sb;
  r.num = r.num * sa + o.num * sb;
  r.mx = mn;
}

template <bool kBf16>
__global__ void __launch_bounds__(kWideThreads) k_compress_wide(CompressArgs a) {
  constexpr int VW = kBf16 ? 8 : 4;        // channels per 16-byte load
  __shared__ float part[kWideThreads * VW * 3];   // [group][field][d]
  __shared__ float red[kWideThreads / 64];
  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int m = a.m;
  const int d = a.d;
  const bool overlap = a.kv_prev != nullptr;
  const int64_t gblk = a.t0 / m + j;
  if (!a.pg.tab && (int64_t)(a.T / m) - j > a.cap) return;   // as k_compress
  const bool has_prev = overlap && gblk > 0;
  const int L = d / VW;                    // lanes per slot group
  const int G = kWideThreads / L;          // slot groups
  const int t = threadIdx.x;
  const int grp = t / L;
  const int c0 = (t % L) * VW;
  // slot index space: overlap = previous-role rows 0..m-1 then current rows
  // 0..m-1 (the bias rows' order); no overlap = current rows 0..m-1
  const int nsl = overlap ? 2 * m : m;
  const int spg = (nsl + G - 1) / G;
  const int s_beg = grp * spg;
  const int s_end = min(nsl, s_beg + spg);
  const int64_t rbase = ((int64_t)b * a.T + (int64_t)j * m) * d + c0;
  Acc acc[VW];
#pragma unroll
  for (int v = 0; v < VW; v++) acc[v] = Acc{-INFINITY, 0.0f, 0.0f};
  for (int s0 = s_beg; s0 < s_end; s0 += kWideUnroll) {
    u32x4 kv[kWideUnroll], gt[kWideUnroll];
    f32x4 bs[kWideUnroll][VW / 4];
#pragma unroll
    for (int u = 0; u < kWideUnroll; u++) {
      const int sl = s0 + u < s_end ? s0 + u : s_end - 1;   // clamped: a real slot
      const bool prev = overlap && sl < m;
      const int tok = prev ? sl : (overlap ? sl - m : sl);
      const size_t idx = (size_t)(rbase + (int64_t)tok * d);
      const void* kvp = prev ? a.kv_prev : a.kv_cur;
      const void* gp = prev ? a.gate_prev : a.gate_cur;
      kv[u] = kBf16 ? *(const u32x4*)((const uint16_t*)kvp + idx) : *(const u32x4*)((const float*)kvp + idx);
      gt[u] = gp ? (kBf16 ? *(const u32x4*)((const uint16_t*)gp + idx) : *(const u32x4*)((const float*)gp + idx))
                 : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int h = 0; h < VW / 4; h++)
        bs[u][h] = a.bias ? *(const f32x4*)(a.bias + (size_t)sl * d + c0 + 4 * h)
                          : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    // the chunk's slots folded at once: its max first, then one exponential
    // per slot (base 2) against the new running max, one rescale per chunk
    bool ok[kWideUnroll];
#pragma unroll
    for (int u = 0; u < kWideUnroll; u++) {
      const int sl = s0 + u;
      ok[u] = sl < s_end && !(overlap && sl < m && !has_prev);   // block 0: no previous rows
    }
#pragma unroll
    for (int v = 0; v < VW; v++) {
      float x[kWideUnroll], z[kWideUnroll];
      float mc = -INFINITY;
#pragma unroll
      for (int u = 0; u < kWideUnroll; u++) {
        if (kBf16) {
          const uint32_t wk = kv[u][v / 2], wg = gt[u][v / 2];
          x[u] = bf16_bits_to_f32((v & 1) ? (wk >> 16) : (wk & 0xFFFFu));
          z[u] = bf16_bits_to_f32((v & 1) ? (wg >> 16) : (wg & 0xFFFFu));
        } else {
          x[u] = __uint_as_float(kv[u][v]);
          z[u] = __uint_as_float(gt[u][v]);
        }
        z[u] += bs[u][v / 4][v % 4];
        mc = ok[u] ? fmaxf(mc, z[u]) : mc;
      }
      if (mc == -INFINITY) continue;       // no slot of this chunk
      Acc& s = acc[v];
      const float mn = fmaxf(s.mx, mc);
      const float mn2 = mn * kLog2eC;
      const float r = s.mx == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(s.mx, kLog2eC, -mn2));
      float se = 0.0f, sev = 0.0f;
#pragma unroll
      for (int u = 0; u < kWideUnroll; u++) {
        const float e = ok[u] ? __builtin_amdgcn_exp2f(fmaf(z[u], kLog2eC, -mn2)) : 0.0f;
        se += e;
        sev = fmaf(e, x[u], sev);
      }
      s.den = fmaf(s.den, r, se);
      s.num = fmaf(s.num, r, sev);
      s.mx = mn;
    }
  }
#pragma unroll
  for (int v = 0; v < VW; v++) {
    part[(grp * 3 + 0) * d + c0 + v] = acc[v].mx;
    part[(grp * 3 + 1) * d + c0 + v] = acc[v].den;
    part[(grp * 3 + 2) * d + c0 + v] = acc[v].num;
  }
  __syncthreads();
  float y[1024 / kWideThreads];
#pragma unroll
  for (int q = 0; q < 1024 / kWideThreads; q++) {
    const int c = t + q * kWideThreads;
    y[q] = 0.0f;
    if (c >= d) continue;
    Acc r{part[c], part[d + c], part[2 * d + c]};
    for (int gg = 1; gg < G; gg++)
      acc_merge(r, Acc{part[(gg * 3) * d + c], part[(gg * 3 + 1) * d + c], part[(gg * 3 + 2) * d + c]});
    y[q] = r.num / r.den;
  }
  finish_entry<kWideThreads>(a, y, b, gblk, red);
}

// Whether the wide kernel takes a call: blocks of at least 32 slots, rows
// that split into 16-byte lanes evenly over a power-of-two lane count.
static bool compress_wide(const CompressArgs& a) {
  const int vw = a.in_bf16 ? 8 : 4;
  if (a.m < 32 || a.d % vw != 0 || a.d > 1024) return false;
  // 16-byte loads: every input must start on a 16-byte boundary
  const uintptr_t any = (uintptr_t)a.kv_cur | (uintptr_t)a.gate_cur | (uintptr_t)a.kv_prev |
                        (uintptr_t)a.gate_prev | (uintptr_t)a.bias;
  if (any & 15) return false;
  const int L = a.d / vw;
  return L <= kWideThreads && (L & (L - 1)) == 0;
}

// State of sequence b: float [2][3][d] = (accumulator k, field: max,
// denominator, numerator, channel); accumulator 0 pools the block of the
// current token, accumulator 1 the previous-role rows of that block (they
// belong to the next block's entry).
template <bool kBf16>
__device__ __forceinline__ void append_one(const CompressArgs& a, int b) {
  __shared__ float red[kCompThreads / 64];
  const int64_t p = a.apos[b];
  if (p < 0) return;                       // uniform: the sequence is idle
  const int m = a.m;
  const int d = a.d;
  const bool overlap = a.kv_prev != nullptr;
  const int u = (int)(p & (m - 1));        // slot of the token in its block (m = 2^k)
  const int64_t blk = p / m;
  const int boff = overlap ? m : 0;
  float* st = a.state ? a.state + (size_t)b * 6 * d : nullptr;
  const float* sr = st ? st : g_zero_row;  // read side (zeros without a state)
  const int sd = st ? d : 0;
  float y[kMaxChan];
#pragma unroll
  for (int q = 0; q < kMaxChan; q++) {
    const int c = threadIdx.x + q * kCompThreads;
    y[q] = 0.0f;
    if (c >= d) continue;
    // every load first, unconditionally (absent inputs read the zero row)
    const size_t ti = (size_t)b * d + c;
    const float kv = ldt<kBf16>(a.kv_cur, ti);
    const float g = a.gate_cur ? ldt<kBf16>(a.gate_cur, ti) : ldt<kBf16>(g_zero_row, c);
    const float bc = (a.bias ? a.bias + (size_t)(boff + u) * d : g_zero_row)[c];
    const float kvp = ldt<kBf16>(overlap ? a.kv_prev : g_zero_row, overlap ? ti : (size_t)c);
    const float gpv = ldt<kBf16>(a.gate_prev ? a.gate_prev : g_zero_row, a.gate_prev ? ti : (size_t)c);
    const float bp = (a.bias && overlap ? a.bias + (size_t)u * d : g_zero_row)[c];
    Acc s0{sr[c], sr[sd + c], sr[2 * sd + c]};
    Acc s1{sr[3 * sd + c], sr[4 * sd + c], sr[5 * sd + c]};
    if (u == 0) {
      // a new block: its entry starts from the previous-role rows pooled
      // during the block before (block 0 has none)
      if (!(overlap && blk > 0)) s1 = Acc{-INFINITY, 0.0f, 0.0f};
      s0 = s1;
      s1 = Acc{-INFINITY, 0.0f, 0.0f};
    }
    acc_add(s0, g + bc, kv);
    if (overlap) acc_add(s1, gpv + bp, kvp);
    y[q] = s0.num / s0.den;
    if (st) {
      st[c] = s0.mx;
      st[d + c] = s0.den;
      st[2 * d + c] = s0.num;
      st[3 * d + c] = s1.mx;
      st[4 * d + c] = s1.den;
      st[5 * d + c] = s1.num;
    }
  }
  if (u != m - 1 || a.no_store) return;    // uniform: no entry to store
  // a block past the sequence's pages is not stored
  if (a.pg.tab && (blk >> a.pg.psh) >= a.pg.tab_ld) return;
  finish_entry<kCompThreads>(a, y, b, blk, red);
}

template <bool kBf16>
__global__ void __launch_bounds__(kCompThreads) k_append(CompressArgs a) {
  append_one<kBf16>(a, blockIdx.x);
}

// Several appends in one launch: workgroup (b, j) runs sequence b of append
// j (the appends touch disjoint states and cache rows).
__global__ void __launch_bounds__(kCompThreads) k_append_batch(AppendBatch ab) {
  const int j = blockIdx.y;
  const CompressArgs& a = ab.c[j];
  if ((int)blockIdx.x >= a.B) return;
  if (a.in_bf16)
    append_one<true>(a, blockIdx.x);
  else
    append_one<false>(a, blockIdx.x);
}

hipError_t launch_append_batch(const AppendBatch& ab, hipStream_t st) {
  int bmax = 0;
  for (int j = 0; j < ab.n; j++) bmax = ab.c[j].B > bmax ? ab.c[j].B : bmax;
  if (ab.n == 0 || bmax == 0) return hipSuccess;
  hipLaunchKernelGGL(k_append_batch, dim3(bmax, ab.n), dim3(kCompThreads), 0, st, ab);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.apos) {
    if (a.in_bf16)
      hipLaunchKernelGGL(k_append<true>, dim3(a.B), dim3(kCompThreads), 0, st, a);
    else
      hipLaunchKernelGGL(k_append<false>, dim3(a.B), dim3(kCompThreads), 0, st, a);
    return hipGetLastError();
  }
  const int nb = a.T / a.m;
  if (nb == 0) return hipSuccess;
  if (compress_wide(a)) {
    if (a.in_bf16)
      hipLaunchKernelGGL(k_compress_wide<true>, dim3(nb, a.B), dim3(kWideThreads), 0, st, a);
    else
      hipLaunchKernelGGL(k_compress_wide<false>, dim3(nb, a.B), dim3(kWideThreads), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_compress, dim3(nb, a.B), dim3(kCompThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace v4a
