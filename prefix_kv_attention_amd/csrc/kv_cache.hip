// Cache writes and the q8_0 dequantisation hook, gfx950.
//
// Once a chunk's step is done its K/V rows are written into the cache, and later
// chunks read them as part of the fixed prefix ("train: walk the window", What it
// is). The storage is F16 or q8_0 (same page, Contents); V is token-major like K,
// so its blocks of 32 run along head_dim (approval comment). bf16 caches are a copy.
//
// The q8_0 block format and the conversions are in pka_device.hpp (q8_0_block,
// to_cache16); the fused forward + append of attn_fwd.hip uses the same functions.
// These kernels move a few MiB and are bound by HBM latency and launch overhead.
#include "pka_device.hpp"

namespace pka {
namespace {

// One thread per append item (a q8_0 block of 32 values, or 8 values for F16 /
// BF16) of all (window, KV head) units.
template <int CT, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int64_t per_unit = append_items<CT, D>(p.C);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t bh = idx / per_unit;
  if (bh * p.C >= p.rows) return;           // rows = B * Hkv * C
  const int64_t it = idx - bh * per_unit;
  const int64_t crow0 = bh * p.cap + window_prefix(p.plens, (int)(bh / p.Hkv), p.P);
  append_item<CT, D>(it, p.C, p.k + bh * p.C * D, p.v + bh * p.C * D, p.ck, p.cv, p.cks,
                     p.cvs, crow0);
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
  const u32x2 c = *reinterpret_cast<const u32x2*>(src);
  RawRow8 raw;
  raw.w = u32x4{c.x, c.y, (uint32_t)(is_v ? p.cvs : p.cks)[crow * (p.D / 32) + c8 / 4], 0u};
  // The same conversion the attention kernels apply when they stage a q8_0 tile:
  // dequant8_q8_0, and for the bf16 output to_bf16x8 (the MFMA operand bits).
  float x[8];
  dequant8_q8_0(raw, x);
  const int64_t out = (is_v ? n * 8 : 0) + orow * p.D + c8 * 8;
  f32x4* of = reinterpret_cast<f32x4*>(p.out_f32 + out);
  of[0] = f32x4{x[0], x[1], x[2], x[3]};
  of[1] = f32x4{x[4], x[5], x[6], x[7]};
  if (p.out_bf16) *reinterpret_cast<u32x4*>(p.out_bf16 + out) = to_bf16x8<kQ8>(raw, true);
}

}  // namespace

template <int CT, int D>
void launch_append_t(const AppendParams& p, hipStream_t s) {
  const int64_t threads = p.rows / p.C * append_items<CT, D>(p.C);
  hipLaunchKernelGGL((append_kernel<CT, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, s, p);
}

hipError_t launch_append(const AppendParams& p, int cache_type, hipStream_t s) {
  prof_begin(PKA_KERNEL_APPEND, s);
  if (p.D == 128) {
    if (cache_type == kQ8) launch_append_t<kQ8, 128>(p, s);
    else if (cache_type == kF16) launch_append_t<kF16, 128>(p, s);
    else launch_append_t<kBF16, 128>(p, s);
  } else {
    if (cache_type == kQ8) launch_append_t<kQ8, 64>(p, s);
    else if (cache_type == kF16) launch_append_t<kF16, 64>(p, s);
    else launch_append_t<kBF16, 64>(p, s);
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
