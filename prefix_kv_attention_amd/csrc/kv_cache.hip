// Cache writes and the q8_0 dequantisation hook, gfx950.
//
// After a chunk is trained it is re-decoded into the cache so the next chunk reads
// it as part of the frozen prefix ("train: walk the window", What it is). The cache
// holds F16 or q8_0 constants (same page, Contents) and V is cached untransposed so
// it can be quantised along head_dim (approval comment). bf16 caches are a copy.
//
// q8_0 block (32 consecutive values of one token row along head_dim):
//   amax = max|x|; d = amax / 127 (IEEE fp32 division; this library is built without
//   fast-math, so '/' is correctly rounded); scale = fp16(d) (RNE);
//   code = clamp(round_half_away_from_zero(x / d), -127, 127) using the fp32 d;
//   amax == 0 stores scale 0 and codes 0. Dequantised value = f32(scale) * code,
//   exact in fp32.
// These kernels move a few MiB and are bound by HBM latency and launch overhead.
#include "pka_device.hpp"

namespace pka {
namespace {

// One thread per 32-value block; K blocks first, then V blocks.
template <int D>
__global__ __launch_bounds__(256) void append_q8_0_kernel(AppendParams p) {
  constexpr int NB = D / 32;
  const int64_t nblk = p.rows * NB;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= 2 * nblk) return;
  const bool is_v = idx >= nblk;
  const int64_t i = is_v ? idx - nblk : idx;
  const int64_t row = i / NB;           // (b*Hkv + kv) * C + t
  const int blk = (int)(i % NB);
  const int64_t bh = row / p.C, tok = row % p.C;
  const uint16_t* src = (is_v ? p.v : p.k) + row * D + blk * 32;

  float x[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 w = reinterpret_cast<const u32x4*>(src)[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[c * 8 + 2 * e] = bf16_to_f32(w[e] & 0xffffu);
      x[c * 8 + 2 * e + 1] = bf16_to_f32(w[e] >> 16);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
  const float d = amax / 127.0f;
  u32x4 q[2];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int code = 0;
      if (d != 0.f) {
        const float r = roundf(x[c * 4 + e] / d);  // halves away from zero
        code = (int)fminf(fmaxf(r, -127.f), 127.f);
      }
      w |= (uint32_t)(code & 0xff) << (8 * e);
    }
    q[c >> 2][c & 3] = w;
  }
  const int64_t crow = bh * p.cap + window_prefix(p.plens, (int)(bh / p.Hkv), p.P) + tok;
  int8_t* dst = static_cast<int8_t*>(is_v ? p.cv : p.ck) + crow * D + blk * 32;
  reinterpret_cast<u32x4*>(dst)[0] = q[0];
  reinterpret_cast<u32x4*>(dst)[1] = q[1];
  (is_v ? p.cvs : p.cks)[crow * NB + blk] = f32_to_f16_bits(d);
}

// One thread per 8 values; F16 converts (RNE), BF16 copies.
template <int CT>
__global__ __launch_bounds__(256) void append_16_kernel(AppendParams p) {
  const int CHK = p.D / 8;
  const int64_t n = p.rows * CHK;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= 2 * n) return;
  const bool is_v = idx >= n;
  const int64_t i = is_v ? idx - n : idx;
  const int64_t row = i / CHK;
  const int c8 = (int)(i % CHK);
  const int64_t bh = row / p.C, tok = row % p.C;
  const u32x4 w = *reinterpret_cast<const u32x4*>((is_v ? p.v : p.k) + row * p.D + c8 * 8);
  u32x4 o;
  if constexpr (CT == kF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)f32_to_f16_bits(bf16_to_f32(w[e] & 0xffffu)) |
             ((uint32_t)f32_to_f16_bits(bf16_to_f32(w[e] >> 16)) << 16);
  } else {
    o = w;
  }
  const int64_t crow = bh * p.cap + window_prefix(p.plens, (int)(bh / p.Hkv), p.P) + tok;
  *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(is_v ? p.cv : p.ck) + crow * p.D + c8 * 8) = o;
}

// One thread per 8 values of K or V rows [row0, row0 + rows).
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(DequantParams p) {
  const int CHK = p.D / 8;
  const int64_t n = p.BH * p.rows * CHK;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= 2 * n) return;
  const bool is_v = idx >= n;
  const int64_t i = is_v ? idx - n : idx;
  const int64_t orow = i / CHK;            // bh * rows + r
  const int c8 = (int)(i % CHK);
  const int64_t bh = orow / p.rows, r = orow % p.rows;
  const int64_t crow = bh * p.cap + p.row0 + r;
  const int8_t* src = (is_v ? p.cv : p.ck) + crow * p.D + c8 * 8;
  const float d = f16_to_f32((is_v ? p.cvs : p.cks)[crow * (p.D / 32) + c8 / 4]);
  const u32x2 c = *reinterpret_cast<const u32x2*>(src);
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = e < 4 ? c.x : c.y;
    x[e] = d * (float)(int8_t)((w >> (8 * (e & 3))) & 0xff);
  }
  const int64_t out = (is_v ? n * 8 : 0) + orow * p.D + c8 * 8;
  f32x4* of = reinterpret_cast<f32x4*>(p.out_f32 + out);
  of[0] = f32x4{x[0], x[1], x[2], x[3]};
  of[1] = f32x4{x[4], x[5], x[6], x[7]};
  if (p.out_bf16) {
    u32x4 o = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
               pack_bf16(x[6], x[7])};
    *reinterpret_cast<u32x4*>(p.out_bf16 + out) = o;
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int cache_type, hipStream_t s) {
  prof_begin(PKA_KERNEL_APPEND, s);
  if (cache_type == kQ8) {
    const int64_t threads = 2 * p.rows * (p.D / 32);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (p.D == 128)
      hipLaunchKernelGGL(append_q8_0_kernel<128>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(append_q8_0_kernel<64>, grid, dim3(256), 0, s, p);
  } else {
    const int64_t threads = 2 * p.rows * (p.D / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (cache_type == kF16)
      hipLaunchKernelGGL(append_16_kernel<kF16>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(append_16_kernel<kBF16>, grid, dim3(256), 0, s, p);
  }
  prof_end(PKA_KERNEL_APPEND, s);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantParams& p, hipStream_t s) {
  const int64_t threads = 2 * p.BH * p.rows * (p.D / 8);
  prof_begin(PKA_KERNEL_DEQUANT, s);
  hipLaunchKernelGGL(dequant_q8_0_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, s, p);
  prof_end(PKA_KERNEL_DEQUANT, s);
  return hipGetLastError();
}

}  // namespace pka
