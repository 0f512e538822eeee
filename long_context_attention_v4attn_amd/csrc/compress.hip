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
#include "common.hpp"
#include "kernels.hpp"

namespace v4a {

constexpr int kCompThreads = 256;
constexpr int kMaxChan = 4;                // d <= 1024

__device__ __forceinline__ float ld(const void* p, int bf16, size_t i) {
  return load_as_f32(p, bf16, i);
}

// kAppend: a decode step ([Notes §11] state cache): one workgroup per
// sequence b and one new token at position p = apos[b].  The token's rows
// join the compressor tails (ring rows p mod t_rows); when the token completes
// block i = (p + 1) / m - 1, the block is pooled like any other: its current
// rows are tail rows except the token itself (read from the input), its
// previous-role rows (tokens of block i - 1) are tail rows.  With t_rows >= 2m
// (>= m without overlap) no row read here is the row the token writes.
template <bool kAppend>
__global__ void __launch_bounds__(kCompThreads) k_compress(CompressArgs a) {
  __shared__ float red[kCompThreads / 64];
  const int m = a.m;
  const int d = a.d;
  const bool overlap = a.kv_prev != nullptr;
  int b, j = 0;
  int64_t gblk, p = 0;
  if (kAppend) {
    b = blockIdx.x;
    p = a.apos[b];
    if (p < 0) return;
    const size_t di = ((size_t)b * a.t_rows + (size_t)(p % a.t_rows)) * d;
    const size_t si = (size_t)b * d;
    auto keep = [&](void* dst, const void* src) {
      if (!dst || !src) return;
      for (int c = threadIdx.x; c < d; c += kCompThreads) {
        if (a.in_bf16) ((uint16_t*)dst)[di + c] = ((const uint16_t*)src)[si + c];
        else ((float*)dst)[di + c] = ((const float*)src)[si + c];
      }
    };
    keep(a.t_kv_cur, a.kv_cur);
    keep(a.t_gate_cur, a.gate_cur);
    keep(a.t_kv_prev, a.kv_prev);
    keep(a.t_gate_prev, a.gate_prev);
    if ((p + 1) % m != 0) return;          // uniform: the block is not complete
    gblk = (p + 1) / m - 1;
    // a block past the sequence's pages is not stored
    if (a.pg.tab && (gblk >> a.pg.psh) >= a.pg.tab_ld) return;
  } else {
    j = blockIdx.x;                        // block within the call
    b = blockIdx.y;
    gblk = a.t0 / m + j;                   // global block index
    // a call that produces more than cap ring entries keeps the last cap of
    // them: an earlier block whose ring row a later block of this call also
    // writes is skipped (concurrent writes to one row would race)
    if (!a.pg.tab && (int64_t)(a.T / m) - j > a.cap) return;
  }
  const bool has_prev = overlap && gblk > 0;
  const int64_t rbase = ((int64_t)b * a.T + (int64_t)j * m) * d;   // row m*j of this call
  // slot sources: the call's rows, or (append) tail rows and the token
  auto prev_idx = [&](int u, int c) -> size_t {
    if (!kAppend) return rbase + (int64_t)u * d + c;
    const int64_t t = (gblk - 1) * m + u;
    return ((size_t)b * a.t_rows + (size_t)(t % a.t_rows)) * d + c;
  };
  const void* kv_prev = kAppend ? a.t_kv_prev : a.kv_prev;
  const void* gate_prev = kAppend ? (a.gate_prev ? a.t_gate_prev : nullptr) : a.gate_prev;

  float y[kMaxChan];
#pragma unroll
  for (int q = 0; q < kMaxChan; q++) {
    const int c = threadIdx.x + q * kCompThreads;
    y[q] = 0.0f;
    if (c >= d) continue;
    float mx = -INFINITY, den = 0.0f, num = 0.0f;
    auto add = [&](float z, float v) {
      if (z > mx) {
        float sc = expf(mx - z);           // mx = -inf -> 0
        den = den * sc + 1.0f;
        num = num * sc + v;
        mx = z;
      } else {
        float e = expf(z - mx);
        den += e;
        num += e * v;
      }
    };
    if (has_prev) {
      for (int u = 0; u < m; u++) {
        size_t idx = prev_idx(u, c);
        float z = (gate_prev ? ld(gate_prev, a.in_bf16, idx) : 0.0f) +
                  (a.bias ? a.bias[(size_t)u * d + c] : 0.0f);
        add(z, ld(kv_prev, a.in_bf16, idx));
      }
    }
    const int boff = overlap ? m : 0;
    for (int u = 0; u < m; u++) {
      const void* kvp = a.kv_cur;
      const void* gp = a.gate_cur;
      size_t idx = rbase + (int64_t)u * d + c;
      if (kAppend) {
        const int64_t t = gblk * m + u;
        if (t == p) {
          idx = (size_t)b * d + c;
        } else {
          kvp = a.t_kv_cur;
          gp = a.gate_cur ? a.t_gate_cur : nullptr;
          idx = ((size_t)b * a.t_rows + (size_t)(t % a.t_rows)) * d + c;
        }
      }
      float z = (gp ? ld(gp, a.in_bf16, idx) : 0.0f) +
                (a.bias ? a.bias[(size_t)(boff + u) * d + c] : 0.0f);
      add(z, ld(kvp, a.in_bf16, idx));
    }
    y[q] = num / den;
  }

  const int64_t orow = a.pg.tab ? page_row(a.pg, b, gblk) : (int64_t)b * a.cap + (gblk % a.cap);
  if (a.out_kind == 0 && (a.nr_gamma || a.nr_inv)) {
    // [Notes §9] KV-entry RMSNorm over the d channels, then RoPE of the last
    // d - d_nope channels at the entry's position (its block's last token):
    // adjacent channels pair up, and since d_nope and 256 are even a pair is
    // two adjacent lanes of one wave
    if (a.nr_gamma) {
      float ss = 0.0f;
#pragma unroll
      for (int q = 0; q < kMaxChan; q++) ss += y[q] * y[q];   // y = 0 past d
      ss = wave_sum(ss);
      __syncthreads();                     // red is free
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
      __syncthreads();
      ss = red[0];
      for (int w = 1; w < kCompThreads / 64; w++) ss += red[w];
      __syncthreads();                     // red is reused below
      const float r = 1.0f / sqrtf(ss / (float)d + a.nr_eps);
#pragma unroll
      for (int q = 0; q < kMaxChan; q++) {
        const int c = threadIdx.x + q * kCompThreads;
        if (c < d) y[q] = y[q] * r * a.nr_gamma[c];
      }
    }
    if (a.nr_inv) {
      const float pf = (float)(gblk * m + m - 1);
#pragma unroll
      for (int q = 0; q < kMaxChan; q++) {
        const int c = threadIdx.x + q * kCompThreads;
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
      for (int q = 0; q < kMaxChan; q++) {
        const int c = threadIdx.x + q * kCompThreads;
        if (c >= d) continue;
        if (c < dn) ((float*)a.o_a)[orow * dn + c] = y[q];
        else ((float*)a.o_b)[orow * dr + (c - dn)] = y[q];
      }
      return;
    }
    // FP8 entry: amax over the non-RoPE channels
    float am = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxChan; q++) {
      const int c = threadIdx.x + q * kCompThreads;
      if (c < dn) am = fmaxf(am, fabsf(y[q]));
    }
    am = wave_max(am);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    am = red[0];
    for (int w = 1; w < kCompThreads / 64; w++) am = fmaxf(am, red[w]);
    const float s = am > 0.0f ? __fdiv_rn(am, kE4M3Max) : 1.0f;
#pragma unroll
    for (int q = 0; q < kMaxChan; q++) {
      const int c = threadIdx.x + q * kCompThreads;
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
    for (int q = 0; q < kMaxChan; q++) {
      const int c = threadIdx.x + q * kCompThreads;
      if (c < d) ((float*)a.o_a)[orow * d + c] = y[q];
    }
    return;
  }
  // MXFP4: d % 32 == 0, so a group of 32 channels is 32 consecutive lanes
#pragma unroll
  for (int q = 0; q < kMaxChan; q++) {
    const int c = threadIdx.x + q * kCompThreads;
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

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.apos) {
    hipLaunchKernelGGL(k_compress<true>, dim3(a.B), dim3(kCompThreads), 0, st, a);
    return hipGetLastError();
  }
  const int nb = a.T / a.m;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(k_compress<false>, dim3(nb, a.B), dim3(kCompThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace v4a
