// Forward of chunk attention against a frozen prefix cache, gfx950.
//
// Computes, for every chunk query row, softmax attention over the cached context
// rows 0..P-1 plus the chunk's own keys 0..i, writing O and the natural-log LSE
// ("Context-Frozen Training", The Solution, Phase 2: the decision tokens run
// against the frozen KV cache; "train: walk the window", What it is: each chunk
// reads the cached prefix as constants).
//
// Design (MI355X):
//  * GQA packing: one workgroup serves 128 packed rows of one (window, KV head);
//    packed row r is token r / G of query head kv*G + r % G, so all query heads
//    that share a KV head read each staged K/V tile from LDS.
//  * Each wave owns 32 rows. Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16, so lane l holds all scores of query row l % 32 for
//    16 keys: the online-softmax row max / row sum need one cross-lane exchange
//    (lane l <-> l^32) per tile, and the running max, sum and rescale factor are
//    per-lane scalars.
//  * O^T += V^T P^T reuses the S^T registers (converted to bf16) directly as the
//    MFMA B operand; V^T is staged in LDS with the matching key permutation.
//  * The key sequence [cache rows ; chunk rows] is streamed in 64-key tiles;
//    F16 / q8_0 cache rows are converted to bf16 while staging to LDS (dequantised
//    on load). Only tiles that cross the causal diagonal are masked.
//  * When (window, KV head, row block) units are too few to fill 256 CUs, the key
//    tiles are split over several workgroups; partial (O, LSE) are merged by
//    fwd_combine in a fixed order (deterministic).
//  * Workgroups are renumbered so each XCD works on a contiguous range of units and
//    the K/V tiles they share stay in that XCD's L2.
#include "pka_device.hpp"

namespace pka {
namespace {

constexpr int BN = kKeysPerTile;

template <int D>
struct FwdSmem {
  static constexpr int KS = D + 8;   // row stride of K (bf16 elements)
  static constexpr int VT = BN + 8;  // row stride of V^T
  uint16_t k[BN * KS];
  uint16_t vt[D * VT];
};

__device__ __forceinline__ uint32_t elem16(const u32x4& w, int e) {
  return (w[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
}

template <int D, int CT>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  __shared__ FwdSmem<D> sm;
  constexpr int KS = FwdSmem<D>::KS;
  constexpr int VT = FwdSmem<D>::VT;
  constexpr int NKS = D / 16;           // k-steps over head_dim
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int CH = D / 8;             // 8-value chunks per row
  constexpr int NTASK = (BN / 4) * CH;  // staging tasks: 4 keys x 8 values

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  const int n_rb = p.plan.n_rb, S = p.plan.n_split;
  const int L = xcd_logical_id(blockIdx.x, p.plan.nblk);
  const int rb = L % n_rb;
  const int split = (L / n_rb) % S;
  const int grp = L / (n_rb * S);
  const int b = grp / p.Hkv, kv = grp % p.Hkv;
  const int G = p.G;
  const int64_t C = p.C, P = p.P;
  const int rows = G * (int)C;

  const int r = rb * kRowsPerBlock + wave * 32 + l32;
  const bool row_ok = r < rows;
  const int rr = row_ok ? r : rows - 1;
  const int t = rr / G;
  const int h = kv * G + (rr - t * G);
  const int64_t qrow = ((int64_t)b * p.Hq + h) * C + t;

  const int r_first = rb * kRowsPerBlock;
  const int r_last = min(rows - 1, r_first + kRowsPerBlock - 1);
  const int t_min = r_first / G, t_max = r_last / G;
  const int64_t key_end = P + t_max + 1;
  const int n_tiles = (int)((key_end + BN - 1) / BN);
  const int tb = (int)((int64_t)split * n_tiles / S);
  const int te = (int)((int64_t)(split + 1) * n_tiles / S);

  bf16x8 qreg[NKS];
  {
    const uint16_t* qp = p.q + qrow * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qreg[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }

  const int64_t bh = (int64_t)b * p.Hkv + kv;
  const int64_t cap = p.cache.cap;
  const void* ck;
  const void* cv;
  if constexpr (CT == kQ8) {
    ck = static_cast<const int8_t*>(p.cache.k) + bh * cap * D;
    cv = static_cast<const int8_t*>(p.cache.v) + bh * cap * D;
  } else {
    ck = static_cast<const uint16_t*>(p.cache.k) + bh * cap * D;
    cv = static_cast<const uint16_t*>(p.cache.v) + bh * cap * D;
  }
  const uint16_t* cks = (CT == kQ8) ? p.cache.ks + bh * cap * (D / 32) : nullptr;
  const uint16_t* cvs = (CT == kQ8) ? p.cache.vs + bh * cap * (D / 32) : nullptr;
  const uint16_t* kcb = p.kc + bh * C * D;
  const uint16_t* vcb = p.vc + bh * C * D;

  const bool has_task = tid < NTASK;
  const int kg = tid / CH, dg = tid % CH;
  RawRow8 rk[4], rv[4];
  bool ik[4], iv[4];

  auto issue = [&](int tile) {
    const int64_t j0 = (int64_t)tile * BN + kg * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ik[i] = load_row8<CT, D>(rk[i], ck, cks, kcb, P, C, j0 + i, dg * 8);
      iv[i] = load_row8<CT, D>(rv[i], cv, cvs, vcb, P, C, j0 + i, dg * 8);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&sm.k[(kg * 4 + i) * KS + dg * 8]) = to_bf16x8<CT>(rk[i], ik[i]);
    u32x4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = to_bf16x8<CT>(rv[i], iv[i]);
    const int pos = swap23(kg * 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x2 pr;
      pr.x = elem16(w[0], e) | (elem16(w[1], e) << 16);
      pr.y = elem16(w[2], e) | (elem16(w[3], e) << 16);
      *reinterpret_cast<u32x2*>(&sm.vt[(dg * 8 + e) * VT + pos]) = pr;
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float c = p.scale_log2;
  const int64_t lim = P + t;  // this row may attend keys 0..lim

  if (tb < te && has_task) issue(tb);
  for (int tile = tb; tile < te; ++tile) {
    __syncthreads();
    if (has_task) stage();
    __syncthreads();
    if (tile + 1 < te && has_task) issue(tile + 1);

    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&sm.k[(kb * 32 + l32) * KS + ks * 16 + hf * 8]);
        st[kb] = mfma32(a, qreg[ks], st[kb]);
      }
    }
    const int64_t kbase = (int64_t)tile * BN;
    if (kbase + BN - 1 > P + t_min) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = kbase + kb * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
          if (key > lim) st[kb][i] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, st[kb][i]);
    mt = fmaxf(mt, wave_xor32(mt));
    const float m_new = fmaxf(m, mt);
    const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
    const float alpha = __builtin_amdgcn_exp2f(m * c - mc);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(st[kb][i], c, -mc));
        st[kb][i] = pv;
        ls += pv;
      }
    l = l * alpha + ls;
    m = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kb * 2 + s][e] = (__bf16)st[kb][s * 8 + e];

#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&sm.vt[(db * 32 + l32) * VT + kk * 16 + hf * 8]);
        acc[db] = mfma32(a, pb[kk], acc[db]);
      }
  }

  const float l_tot = l + wave_xor32(l);
  if (!row_ok) return;
  if (S == 1) {
    const float inv = 1.f / l_tot;
    uint16_t* op = p.o + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hf * 4;
        u32x2 w;
        w.x = pack_bf16(acc[db][g4 * 4 + 0] * inv, acc[db][g4 * 4 + 1] * inv);
        w.y = pack_bf16(acc[db][g4 * 4 + 2] * inv, acc[db][g4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d) = w;
      }
    if (hf == 0) p.lse[qrow] = m * p.scale + logf(l_tot);
  } else {
    const int64_t nrow = (int64_t)p.B * p.Hq * C;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* wo = p.ws_o + ((int64_t)split * nrow + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hf * 4;
        f32x4 w = {acc[db][g4 * 4 + 0] * inv, acc[db][g4 * 4 + 1] * inv,
                   acc[db][g4 * 4 + 2] * inv, acc[db][g4 * 4 + 3] * inv};
        *reinterpret_cast<f32x4*>(wo + d) = w;
      }
    if (hf == 0)
      p.ws_lse[(int64_t)split * nrow + qrow] =
          l_tot > 0.f ? m * p.scale + logf(l_tot) : -INFINITY;
  }
}

// Merge of prefix splits: LSE = logsumexp_s LSE_s, O = sum_s exp(LSE_s - LSE) O_s,
// summed in split order.
template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(FwdParams p) {
  constexpr int CH = D / 8;
  const int64_t nrow = (int64_t)p.B * p.Hq * p.C;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / CH;
  const int c8 = (int)(idx % CH);
  if (row >= nrow) return;
  const int S = p.plan.n_split;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, p.ws_lse[s * nrow + row]);
  float sum = 0.f;
  for (int s = 0; s < S; ++s) sum += expf(p.ws_lse[s * nrow + row] - mx);
  const float lse = mx + logf(sum);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float w = expf(p.ws_lse[s * nrow + row] - lse);
    const f32x4* src = reinterpret_cast<const f32x4*>(p.ws_o + (s * nrow + row) * D + c8 * 8);
    const f32x4 a = src[0], bq = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] += w * a[i];
      o[4 + i] += w * bq[i];
    }
  }
  u32x4 out = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]),
               pack_bf16(o[6], o[7])};
  *reinterpret_cast<u32x4*>(p.o + row * D + c8 * 8) = out;
  if (c8 == 0) p.lse[row] = lse;
}

template <int D, int CT>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  prof_begin(PKA_KERNEL_FWD, s);
  hipLaunchKernelGGL((fwd_kernel<D, CT>), dim3(p.plan.nblk), dim3(256), 0, s, p);
  prof_end(PKA_KERNEL_FWD, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.plan.n_split == 1) return e;
  const int64_t threads = (int64_t)p.B * p.Hq * p.C * (D / 8);
  prof_begin(PKA_KERNEL_FWD_COMBINE, s);
  hipLaunchKernelGGL((fwd_combine_kernel<D>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, s, p);
  prof_end(PKA_KERNEL_FWD_COMBINE, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int D, int cache_type, hipStream_t s) {
  if (D == 128) {
    if (cache_type == kF16) return launch_fwd_t<128, kF16>(p, s);
    if (cache_type == kBF16) return launch_fwd_t<128, kBF16>(p, s);
    return launch_fwd_t<128, kQ8>(p, s);
  }
  if (cache_type == kF16) return launch_fwd_t<64, kF16>(p, s);
  if (cache_type == kBF16) return launch_fwd_t<64, kBF16>(p, s);
  return launch_fwd_t<64, kQ8>(p, s);
}

}  // namespace pka
