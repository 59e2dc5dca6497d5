// Backward of chunk attention against a frozen prefix cache, gfx950.
//
// Gradient flows through the chunk only: dQ for the chunk's query rows over every
// key they read (cache and chunk), and dK/dV for the chunk's own C keys. The cached
// rows are stop-gradient constants and get nothing ("Context-Frozen Training",
// The Gradient Signal; "train: walk the window", Why it's a draft: cached prefixes
// are stop-gradient constants; "stop-gradient through context tokens", Known gaps:
// an attention backward that computes gradient for the kept queries only).
//
// Kernels, in launch order on the caller's stream:
//  1. bwd_prep:  delta_i = sum_d dO_id * O_id from the stored bf16 O.
//  2. bwd_dq:    per 128 packed query rows (GQA packing as in the forward), stream
//                the key tiles: S^T = K Q^T, dP^T = V dO^T (MFMA bf16),
//                P = exp2(S*scale*log2e - LSE*log2e), dS = P (dP - delta) in
//                registers, dQ^T += K^T dS^T (MFMA, dS^T registers reused as the B
//                operand). Split over key tiles like the forward when the units
//                are too few; fp32 partials are summed by bwd_dq_reduce in a fixed
//                order.
//  3. bwd_dkdv:  per 128 chunk keys of one (window, KV head), stream the packed
//                query rows of all G heads that can see them (token >= key):
//                S = Q K^T and dP = dO V^T with keys as MFMA columns, then
//                dV^T += dO^T P and dK^T += Q^T dS; the sum over the G heads of a
//                KV head falls out of the packing. No atomics: every output element
//                is owned by one lane.
#include "pka_device.hpp"

namespace pka {
namespace {

constexpr int BN = kKeysPerTile;

__device__ __forceinline__ uint32_t elem16(const u32x4& w, int e) {
  return (w[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
}

// 4 rows x 8 values -> transposed LDS rows dst[(d0+e)*stride + pos .. pos+3].
__device__ __forceinline__ void store_transposed(uint16_t* dst, int stride, int d0,
                                                 int pos, const u32x4 (&w)[4]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u32x2 pr;
    pr.x = elem16(w[0], e) | (elem16(w[1], e) << 16);
    pr.y = elem16(w[2], e) | (elem16(w[3], e) << 16);
    *reinterpret_cast<u32x2*>(&dst[(d0 + e) * stride + pos]) = pr;
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int CH = D / 8;
  const int64_t nrow = (int64_t)p.B * p.Hq * p.C;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / CH;
  const int c8 = (int)(idx % CH);
  float s = 0.f;
  if (row < nrow) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p.o + row * D + c8 * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(p.d_o + row * D + c8 * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      s = fmaf(bf16_to_f32(elem16(a, e)), bf16_to_f32(elem16(g, e)), s);
  }
#pragma unroll
  for (int off = CH / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (row < nrow && c8 == 0) p.delta[row] = s;
}

template <int D>
struct DqSmem {
  static constexpr int KS = D + 8;
  static constexpr int KT = BN + 8;
  uint16_t k[BN * KS];
  uint16_t kt[D * KT];
  uint16_t v[BN * KS];
};

template <int D, int CT>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdParams p) {
  __shared__ DqSmem<D> sm;
  constexpr int KS = DqSmem<D>::KS;
  constexpr int KT = DqSmem<D>::KT;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CH = D / 8;
  constexpr int NTASK = (BN / 4) * CH;

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

  bf16x8 qreg[NKS], oreg[NKS];
  {
    const uint16_t* qp = p.q + qrow * D + hf * 8;
    const uint16_t* gp = p.d_o + qrow * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qreg[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
      oreg[ks] = *reinterpret_cast<const bf16x8*>(gp + ks * 16);
    }
  }
  const float c = p.scale_log2;
  const float lse2 = p.lse[qrow] * kLog2e;
  const float dlt = p.delta[qrow];

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
    u32x4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = to_bf16x8<CT>(rk[i], ik[i]);
      *reinterpret_cast<u32x4*>(&sm.k[(kg * 4 + i) * KS + dg * 8]) = w[i];
      *reinterpret_cast<u32x4*>(&sm.v[(kg * 4 + i) * KS + dg * 8]) = to_bf16x8<CT>(rv[i], iv[i]);
    }
    store_transposed(sm.kt, KT, dg * 8, swap23(kg * 4), w);
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  const int64_t lim = P + t;

  if (tb < te && has_task) issue(tb);
  for (int tile = tb; tile < te; ++tile) {
    __syncthreads();
    if (has_task) stage();
    __syncthreads();
    if (tile + 1 < te && has_task) issue(tile + 1);

    f32x16 st[2], dpt[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x16{};
      dpt[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int off = (kb * 32 + l32) * KS + ks * 16 + hf * 8;
        st[kb] = mfma32(*reinterpret_cast<const bf16x8*>(&sm.k[off]), qreg[ks], st[kb]);
        dpt[kb] = mfma32(*reinterpret_cast<const bf16x8*>(&sm.v[off]), oreg[ks], dpt[kb]);
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
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(st[kb][i], c, -lse2));
        dsb[kb * 2 + (i >> 3)][i & 7] = (__bf16)(pv * (dpt[kb][i] - dlt));
      }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&sm.kt[(db * 32 + l32) * KT + kk * 16 + hf * 8]);
        acc[db] = mfma32(a, dsb[kk], acc[db]);
      }
  }

  if (!row_ok) return;
  const float sc = p.scale;
  if (S == 1) {
    uint16_t* op = p.dq + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hf * 4;
        u32x2 w;
        w.x = pack_bf16(acc[db][g4 * 4 + 0] * sc, acc[db][g4 * 4 + 1] * sc);
        w.y = pack_bf16(acc[db][g4 * 4 + 2] * sc, acc[db][g4 * 4 + 3] * sc);
        *reinterpret_cast<u32x2*>(op + d) = w;
      }
  } else {
    const int64_t nrow = (int64_t)p.B * p.Hq * C;
    float* wo = p.ws_dq + ((int64_t)split * nrow + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hf * 4;
        f32x4 w = {acc[db][g4 * 4 + 0] * sc, acc[db][g4 * 4 + 1] * sc,
                   acc[db][g4 * 4 + 2] * sc, acc[db][g4 * 4 + 3] * sc};
        *reinterpret_cast<f32x4*>(wo + d) = w;
      }
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(BwdParams p) {
  constexpr int CH = D / 8;
  const int64_t nrow = (int64_t)p.B * p.Hq * p.C;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / CH;
  const int c8 = (int)(idx % CH);
  if (row >= nrow) return;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.plan.n_split; ++s) {
    const f32x4* src = reinterpret_cast<const f32x4*>(p.ws_dq + (s * nrow + row) * D + c8 * 8);
    const f32x4 a = src[0], bq = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] += a[i];
      o[4 + i] += bq[i];
    }
  }
  u32x4 out = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]),
               pack_bf16(o[6], o[7])};
  *reinterpret_cast<u32x4*>(p.dq + row * D + c8 * 8) = out;
}

constexpr int BQ = 32;  // packed query rows per dK/dV step

template <int D>
struct DkvSmem {
  static constexpr int QS = D + 8;
  static constexpr int QT = BQ + 8;
  uint16_t q[BQ * QS];
  uint16_t g[BQ * QS];   // dO
  uint16_t qt[D * QT];
  uint16_t gt[D * QT];
  float lse2[BQ];
  float dlt[BQ];
  int tok[BQ];
};

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdParams p) {
  __shared__ DkvSmem<D> sm;
  constexpr int QS = DkvSmem<D>::QS;
  constexpr int QT = DkvSmem<D>::QT;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CH = D / 8;
  constexpr int NT = (BQ / 4) * CH;  // staging tasks per tensor (<= 128)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t C = p.C;
  const int G = p.G;
  const int rows = G * (int)C;
  const int nkb = (int)((C + kDkvKeysPerBlock - 1) / kDkvKeysPerBlock);
  const int L = blockIdx.x;
  const int kblk = L % nkb;
  const int grp = L / nkb;
  const int b = grp / p.Hkv, kv = grp % p.Hkv;
  const int64_t bh = (int64_t)b * p.Hkv + kv;

  const int key = kblk * kDkvKeysPerBlock + wave * 32 + l32;  // chunk index
  const bool key_ok = key < C;
  bf16x8 kreg[NKS], vreg[NKS];
  {
    const uint16_t* kp = p.kc + (bh * C + (key_ok ? key : 0)) * D + hf * 8;
    const uint16_t* vp = p.vc + (bh * C + (key_ok ? key : 0)) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kreg[ks] = *reinterpret_cast<const bf16x8*>(kp + ks * 16);
      vreg[ks] = *reinterpret_cast<const bf16x8*>(vp + ks * 16);
      if (!key_ok) {
        kreg[ks] = bf16x8{};
        vreg[ks] = bf16x8{};
      }
    }
  }
  f32x16 acck[NDB], accv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    acck[db] = f32x16{};
    accv[db] = f32x16{};
  }
  const float c = p.scale_log2;

  // Query rows whose token is >= the block's first key can see some key of it.
  const int r_begin = kblk * kDkvKeysPerBlock * G;
  const bool stages_q = tid < NT;
  const bool stages_g = tid >= 128 && tid < 128 + NT;
  const int task = stages_q ? tid : tid - 128;
  const int rg = task / CH, dg = task % CH;

  for (int r0 = r_begin; r0 < rows; r0 += BQ) {
    __syncthreads();
    if (stages_q || stages_g) {
      const uint16_t* src = stages_q ? p.q : p.d_o;
      u32x4 w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = r0 + rg * 4 + i;
        if (rr < rows) {
          const int tt = rr / G;
          const int hh = kv * G + (rr - tt * G);
          const int64_t row = ((int64_t)b * p.Hq + hh) * C + tt;
          w[i] = *reinterpret_cast<const u32x4*>(src + row * D + dg * 8);
        } else {
          w[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      uint16_t* rowmajor = stages_q ? sm.q : sm.g;
      uint16_t* trans = stages_q ? sm.qt : sm.gt;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(&rowmajor[(rg * 4 + i) * QS + dg * 8]) = w[i];
      store_transposed(trans, QT, dg * 8, swap23(rg * 4), w);
    }
    if (tid < BQ) {
      const int rr = r0 + tid;
      if (rr < rows) {
        const int tt = rr / G;
        const int hh = kv * G + (rr - tt * G);
        const int64_t row = ((int64_t)b * p.Hq + hh) * C + tt;
        sm.lse2[tid] = p.lse[row] * kLog2e;
        sm.dlt[tid] = p.delta[row];
        sm.tok[tid] = tt;
      } else {
        sm.lse2[tid] = 0.f;
        sm.dlt[tid] = 0.f;
        sm.tok[tid] = -1;
      }
    }
    __syncthreads();

    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int off = l32 * QS + ks * 16 + hf * 8;
      s = mfma32(*reinterpret_cast<const bf16x8*>(&sm.q[off]), kreg[ks], s);
      dp = mfma32(*reinterpret_cast<const bf16x8*>(&sm.g[off]), vreg[ks], dp);
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qi = (i >> 2) * 8 + hf * 4 + (i & 3);
      const float pv = (key <= sm.tok[qi])
                           ? __builtin_amdgcn_exp2f(fmaf(s[i], c, -sm.lse2[qi]))
                           : 0.f;
      pb[i >> 3][i & 7] = (__bf16)pv;
      dsb[i >> 3][i & 7] = (__bf16)(pv * (dp[i] - sm.dlt[qi]));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const int off = (db * 32 + l32) * QT + ss * 16 + hf * 8;
        accv[db] = mfma32(*reinterpret_cast<const bf16x8*>(&sm.gt[off]), pb[ss], accv[db]);
        acck[db] = mfma32(*reinterpret_cast<const bf16x8*>(&sm.qt[off]), dsb[ss], acck[db]);
      }
  }

  if (!key_ok) return;
  const float sc = p.scale;
  uint16_t* dkp = p.dk + (bh * C + key) * D;
  uint16_t* dvp = p.dv + (bh * C + key) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + g4 * 8 + hf * 4;
      u32x2 wk, wv;
      wk.x = pack_bf16(acck[db][g4 * 4 + 0] * sc, acck[db][g4 * 4 + 1] * sc);
      wk.y = pack_bf16(acck[db][g4 * 4 + 2] * sc, acck[db][g4 * 4 + 3] * sc);
      wv.x = pack_bf16(accv[db][g4 * 4 + 0], accv[db][g4 * 4 + 1]);
      wv.y = pack_bf16(accv[db][g4 * 4 + 2], accv[db][g4 * 4 + 3]);
      *reinterpret_cast<u32x2*>(dkp + d) = wk;
      *reinterpret_cast<u32x2*>(dvp + d) = wv;
    }
}

template <int D, int CT>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
  const int64_t nrow = (int64_t)p.B * p.Hq * p.C;
  const unsigned row_blocks = (unsigned)((nrow * (D / 8) + 255) / 256);
  prof_begin(PKA_KERNEL_BWD_PREP, s);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(row_blocks), dim3(256), 0, s, p);
  prof_end(PKA_KERNEL_BWD_PREP, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  prof_begin(PKA_KERNEL_BWD_DQ, s);
  hipLaunchKernelGGL((bwd_dq_kernel<D, CT>), dim3(p.plan.nblk), dim3(256), 0, s, p);
  prof_end(PKA_KERNEL_BWD_DQ, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const int nkb = (int)((p.C + kDkvKeysPerBlock - 1) / kDkvKeysPerBlock);
  prof_begin(PKA_KERNEL_BWD_DKDV, s);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3(p.B * p.Hkv * nkb), dim3(256), 0, s, p);
  prof_end(PKA_KERNEL_BWD_DKDV, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  if (p.plan.n_split > 1) {
    prof_begin(PKA_KERNEL_BWD_DQ_REDUCE, s);
    hipLaunchKernelGGL((bwd_dq_reduce_kernel<D>), dim3(row_blocks), dim3(256), 0, s, p);
    prof_end(PKA_KERNEL_BWD_DQ_REDUCE, s);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int D, int cache_type, hipStream_t s) {
  if (D == 128) {
    if (cache_type == kF16) return launch_bwd_t<128, kF16>(p, s);
    if (cache_type == kBF16) return launch_bwd_t<128, kBF16>(p, s);
    return launch_bwd_t<128, kQ8>(p, s);
  }
  if (cache_type == kF16) return launch_bwd_t<64, kF16>(p, s);
  if (cache_type == kBF16) return launch_bwd_t<64, kBF16>(p, s);
  return launch_bwd_t<64, kQ8>(p, s);
}

}  // namespace pka
