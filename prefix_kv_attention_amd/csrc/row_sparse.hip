// Row-sparse linear backward, gfx950 ("stop-gradient through context tokens",
// Mechanism): for y = x W^T with the upstream gradient dY read only on the kept rows,
//   dW = dY[keep]^T X[keep]                       (f32 [out][in])
//   dX[keep] = dY[keep] W,  dX[other rows] = 0    (bf16 [N][in])
// Both are dense contractions once the kept rows are gathered, so they run on MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation); the gather is fused into the loads
// that stage the operand tiles in LDS, so no compacted copy of x or dY is made.
//
// Design (MI355X):
//  * One kernel template for both products. A workgroup owns a 128 x 128 output tile
//    and walks the contraction in k-stages of 64 through two LDS buffers (one barrier
//    per stage); the rows of the stage three ahead are loaded into registers while a
//    stage is computed. 4 waves of 64 x 64 (2 x 2 MFMA blocks, up to two workgroups
//    per CU), or 8 waves of 64 x 32 when the grid has at most one tile per CU.
//  * dX is computed transposed, dX^T = W^T dY[keep]^T: its A operand is W^T, read
//    from the row-major W tile with the transposing LDS read; its B operand is a
//    gathered dY row, read as is. The transposing read returns each 16-deep k-step
//    in the order of an MFMA result's registers (bits 2 and 3 of the index
//    exchanged), so the W rows are staged with that exchange applied and both
//    operands see the same k order. Each lane then holds one kept row of dX and
//    stores 4 consecutive features at a time.
//  * dW = dY[keep]^T X[keep] contracts over the kept rows: both operands are gathered
//    rows read with the transposing LDS read, so their k orders agree as they are.
//    Each kept-row index is loaded two stages before the rows it addresses.
//  * dX is zeroed by a streaming fill launched before the dX product, which then
//    writes the kept rows: right for distinct kept rows in any order.
//  * A dX grid of fewer tiles than CUs is split over the output features: fp32
//    partials in the caller's workspace, summed in split order by a reduction that
//    writes the kept rows.
//  * Workgroups are renumbered so each XCD works on a contiguous range of tiles that
//    form a near-square block of the output: the operand rows of the block stay in
//    that XCD's L2 (q_proj at 2048 tokens: HBM fetch of the dX product 70 MB with
//    one tile column per XCD, for 12 MB of operands).
#include <type_traits>

#include "pka_device.hpp"
#include "row_sparse.hpp"

namespace pka {
namespace {

constexpr int BT = kRsTile;     // output tile (both dimensions)
constexpr int BK = kRsStage;    // k-stage
constexpr int SW = BT + 8;      // row stride (elements) of the [k][128] tiles
constexpr int SR = BK + 8;      // row stride of the dX kernel's [row][64] dY tile

enum : int { kDX = 0, kDW = 1 };

template <int MODE>
struct RsLds {
  uint16_t a[2][BK * SW];                          // [k][i]: W rows or gathered dY rows
  uint16_t b[2][MODE == kDX ? BT * SR : BK * SW];  // dX: [row][k] dY; dW: [k][j] x rows
};

// Waves of a workgroup: 2 along i (64 rows each) x BT / (32 JB) along j (JB blocks of
// 32 columns each): JB = 2 gives 4 waves of 64 x 64, JB = 1 gives 8 waves of 64 x 32
// (two per SIMD on the same tile, for grids too small to put two workgroups on a CU).
template <int JB>
constexpr int rs_threads() { return 64 * 2 * (BT / (32 * JB)); }

template <int MODE, int JB>
__global__ __launch_bounds__(rs_threads<JB>()) void row_sparse_kernel(RsParams p) {
  constexpr int RNT = rs_threads<JB>();
  constexpr int CPT = BK * BT / 8 / RNT;   // 16-byte chunks per thread per tile per stage
  __shared__ __align__(16) RsLds<MODE> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int wi = wave & 1, wj = wave >> 1;
  const int jw = wj * 32 * JB;   // this wave's first column of the tile

  // dX^T: i = input feature, j = kept row (position in keep), k = output feature.
  // dW:   i = output feature, j = input feature, k = kept row.
  const int TI = (MODE == kDX ? p.in : p.out) / BT;
  const int TJ = MODE == kDX ? (int)((p.K + BT - 1) / BT) : p.in / BT;
  const int SPL = MODE == kDX ? p.dx_split : 1;   // splits of the contraction
  const int Lg = xcd_logical_id(blockIdx.x, TI * TJ * SPL);
  const int sp = Lg / (TI * TJ);                  // this workgroup's split
  const int L = Lg - sp * TI * TJ;
  // Each XCD's contiguous range of ids walks groups of GM i-tiles across all j-tiles,
  // so the range covers a near-square block of the output and its L2 holds the rows
  // of both operands that the block needs (GM: the largest power of 2 whose square
  // fits in one XCD's share of the tiles, at most TI).
  const int per_xcd = (TI * TJ + kNumXCDs - 1) / kNumXCDs;
  int GM = 1;
  while (GM * 2 <= TI && GM * GM * 4 <= per_xcd) GM *= 2;
  const int group = L / (GM * TJ), first = group * GM;
  const int gsz = min(TI - first, GM);
  const int in_group = L - group * GM * TJ;
  const int i0 = (first + in_group % gsz) * BT, j0 = (in_group / gsz) * BT;
  const int64_t KD = MODE == kDX ? (int64_t)p.out : p.K;   // contraction length
  const int n_all = (int)((KD + BK - 1) / BK);
  const int st0 = (int)((int64_t)sp * n_all / SPL);          // this split's k-stages
  const int n_st = (int)((int64_t)(sp + 1) * n_all / SPL) - st0;

  // Staging: thread tid stages chunks c = tid + s * RNT (s < CPT) of each tile.
  // [k][128] tiles: row c / 16, 8 values at column 8 (c % 16). The dX kernel's dY
  // tile [row][64]: row c / 8, 8 values at column 8 (c % 8). Loads run three stages
  // ahead of the compute into two register sets (set = stage parity): a stage is
  // short (16 MFMAs per wave), so one stage of lead would not cover the latency of a
  // gathered row.
  u32x4 ra[2][CPT], rb[2][CPT];
  bool ok[2][CPT];       // the staged row exists (else zeros are staged). dX: fixed,
                         // in set 0; dW: set by issue() for the stage it loads
  int64_t drow[CPT];     // dX: element offset of each staged dY row (the same rows
                         // j0 + c / 8 in every stage)
  int kidx[2][CPT];      // dW: kept-row indices of the stages to issue (by parity),
                         // loaded two steps before the rows they address
  if constexpr (MODE == kDX) {
#pragma unroll
    for (int s = 0; s < CPT; ++s) {
      const int64_t m = j0 + (tid + s * RNT) / 8;
      int32_t r = m < p.K ? p.keep[m] : -1;
      ok[0][s] = r >= 0 && r < p.N;
      if (!ok[0][s]) r = 0;   // load a valid row; zeros are staged instead
      drow[s] = (int64_t)r * p.out;
    }
  }
  auto load_idx = [&](auto set, int st) {   // dW only
    constexpr int R = decltype(set)::value;
#pragma unroll
    for (int s = 0; s < CPT; ++s) {
      const int64_t k = (int64_t)(st0 + st) * BK + (tid + s * RNT) / 16;
      kidx[R][s] = p.keep[k < p.K ? k : 0];
    }
  };
  auto issue = [&](auto set, int st) {
    constexpr int R = decltype(set)::value;
    const int64_t k0 = (int64_t)(st0 + st) * BK;
#pragma unroll
    for (int s = 0; s < CPT; ++s) {
      const int c = tid + s * RNT;
      const int cc = c % 16;
      if constexpr (MODE == kDX) {
        ra[R][s] = *reinterpret_cast<const u32x4*>(p.w + (k0 + c / 16) * p.in + i0 + cc * 8);
        rb[R][s] = *reinterpret_cast<const u32x4*>(p.dy + drow[s] + k0 + (c % 8) * 8);
      } else {
        int32_t r = kidx[R][s];
        ok[R][s] = k0 + c / 16 < p.K && r >= 0 && r < p.N;
        if (!ok[R][s]) r = 0;
        ra[R][s] = *reinterpret_cast<const u32x4*>(p.dy + (int64_t)r * p.out + i0 + cc * 8);
        rb[R][s] = *reinterpret_cast<const u32x4*>(p.x + (int64_t)r * p.in + j0 + cc * 8);
      }
    }
  };
  auto store = [&](auto set, int buf) {
    constexpr int R = decltype(set)::value;
#pragma unroll
    for (int s = 0; s < CPT; ++s) {
      const int c = tid + s * RNT;
      const int kk = c / 16, cc = c % 16;
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      if constexpr (MODE == kDX) {
        // W row kk at the row the transposing read returns in natural k order
        *reinterpret_cast<u32x4*>(&sm.a[buf][prow(swap23(kk)) * SW + cc * 8]) = ra[R][s];
        *reinterpret_cast<u32x4*>(&sm.b[buf][prow(c / 8) * SR + (c % 8) * 8]) =
            ok[0][s] ? rb[R][s] : z;
      } else {
        *reinterpret_cast<u32x4*>(&sm.a[buf][prow(kk) * SW + cc * 8]) = ok[R][s] ? ra[R][s] : z;
        *reinterpret_cast<u32x4*>(&sm.b[buf][prow(kk) * SW + cc * 8]) = ok[R][s] ? rb[R][s] : z;
      }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  const TrOffsets t_off = tr_lane_offsets<SW>(lane);
  const int b_off = (jw + prow(l32)) * SR + hf * 8;   // dX: B operand rows
  f32x16 acc[2][JB];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) acc[ib][jb] = f32x16{};

  // Prologue: stage 0 into LDS, stages 1 and 2 in registers (sets 1 and 0). Loads
  // past the last stage re-read the last stage (never computed): every step then
  // issues the same loads, and the compiler's waits stay at "all but the newest set"
  // instead of draining every load at the branch that would skip them.
  const int last = n_st - 1;
  if (n_st > 0) {
    if constexpr (MODE == kDW) load_idx(S0{}, 0);
    issue(S0{}, 0);
    if constexpr (MODE == kDW) load_idx(S1{}, min(1, last));
    issue(S1{}, min(1, last));
    store(S0{}, 0);
    if constexpr (MODE == kDW) load_idx(S0{}, min(2, last));
    issue(S0{}, min(2, last));
    if constexpr (MODE == kDW) {
      load_idx(S1{}, min(3, last));
      load_idx(S0{}, min(4, last));
    }
  }
  __syncthreads();
  wait_global_loads();
  // Stage st: compute from LDS buffer st & 1; write stage st + 1 (register set
  // (st + 1) & 1) into the other buffer; load stage st + 3 into the set just freed.
  auto step = [&](auto set_next, int st) {
    const int cur = st & 1;
    const uint16_t* at = sm.a[cur];
    const uint16_t* bt = sm.b[cur];
    bf16x8 av[2][4], bv[JB][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int x = 0; x < 2; ++x) av[x][ks] = lds_tr_operand<SW>(at, t_off, ks * 16, wi * 64 + x * 32);
#pragma unroll
      for (int x = 0; x < JB; ++x) {
        if constexpr (MODE == kDX)
          bv[x][ks] = *reinterpret_cast<const bf16x8*>(&bt[b_off + x * 32 * SR + ks * 16]);
        else
          bv[x][ks] = lds_tr_operand<SW>(bt, t_off, ks * 16, jw + x * 32);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) acc[ib][jb] = mfma32(av[ib][ks], bv[jb][ks], acc[ib][jb]);
    // The other buffer was last read in step st - 1, which every wave has left (the
    // barrier below it); after the last stage this writes rows nobody reads.
    store(set_next, cur ^ 1);
    issue(set_next, min(st + 3, last));
    if constexpr (MODE == kDW) load_idx(set_next, min(st + 5, last));
    __syncthreads();
  };
  int st = 0;
  for (; st + 1 < n_st; st += 2) {
    step(S1{}, st);
    step(S0{}, st + 1);
  }
  if (st < n_st) step(S1{}, st);

  // Register r of block (ib, jb) is row i0 + wi*64 + ib*32 + (r/4)*8 + hf*4 + r%4 of
  // the tile's i range, lane l32 column j0 + jw + jb*32 + l32 of its j range.
  if (MODE == kDX && SPL > 1) {
    // fp32 partials of this split, rows in kept order: [split][K][in]
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int64_t m = j0 + jw + jb * 32 + l32;
      if (m >= p.K) continue;
      float* dst = p.ws + ((int64_t)sp * p.K + m) * p.in + i0 + wi * 64 + hf * 4;
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4*>(dst + ib * 32 + g4 * 8) =
              f32x4{acc[ib][jb][g4 * 4 + 0], acc[ib][jb][g4 * 4 + 1],
                    acc[ib][jb][g4 * 4 + 2], acc[ib][jb][g4 * 4 + 3]};
    }
  } else if constexpr (MODE == kDX) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int64_t m = j0 + jw + jb * 32 + l32;
      if (m >= p.K) continue;
      const int32_t r = p.keep[m];
      if (r < 0 || r >= p.N) continue;
      uint16_t* dst = p.dx + (int64_t)r * p.in + i0 + wi * 64 + hf * 4;
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 v;
          v.x = pack_bf16(acc[ib][jb][g4 * 4 + 0], acc[ib][jb][g4 * 4 + 1]);
          v.y = pack_bf16(acc[ib][jb][g4 * 4 + 2], acc[ib][jb][g4 * 4 + 3]);
          *reinterpret_cast<u32x2*>(dst + ib * 32 + g4 * 8) = v;
        }
    }
  } else {
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        float* dst = p.dw + (int64_t)(i0 + wi * 64 + ib * 32 + hf * 4) * p.in + j0 + jw +
                     jb * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(int64_t)((r / 4) * 8 + r % 4) * p.in] = acc[ib][jb][r];
      }
  }
}

// dX before the product: every row zero (16 bytes per thread). The product then
// writes the kept rows, so rows that are not kept end as zeros whatever the order of
// the kept list (a streaming write of N x in bf16; no search of the list).
__global__ __launch_bounds__(256) void row_sparse_zero_kernel(RsParams p) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.N * (p.in / 8)) return;
  reinterpret_cast<u32x4*>(p.dx)[idx] = u32x4{0u, 0u, 0u, 0u};
}

// dX split over output features: the partials of each kept row summed in split order
// (deterministic), rounded to bf16 and written to its row of dX.
__global__ __launch_bounds__(256) void row_sparse_dx_reduce_kernel(RsParams p) {
  const int ch = p.in / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t m = idx / ch;
  if (m >= p.K) return;
  const int32_t r = p.keep[m];
  if (r < 0 || r >= p.N) return;
  const int c8 = (int)(idx % ch);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < p.dx_split; ++sp) {
    const f32x4* v = reinterpret_cast<const f32x4*>(p.ws + ((int64_t)sp * p.K + m) * p.in + c8 * 8);
    const f32x4 a = v[0], b = v[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] += a[i];
      o[4 + i] += b[i];
    }
  }
  *reinterpret_cast<u32x4*>(p.dx + (int64_t)r * p.in + c8 * 8) =
      u32x4{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]),
            pack_bf16(o[6], o[7])};
}

template <int MODE>
hipError_t launch_product(const RsParams& p, int64_t tiles, hipStream_t s) {
  // Grids of at most one tile per CU run 8 waves per tile (two per SIMD); larger ones
  // 4 waves (up to two workgroups per CU). Measured at 2048 tokens: q_proj dX 26.6 ->
  // 25.0 us and dW 21.8 -> 20.1 us with 8 waves; down_proj dX (384 tiles) 47.6 us with
  // 4 waves against 53.1 us with 8.
  if (tiles <= kNumCUs)
    hipLaunchKernelGGL((row_sparse_kernel<MODE, 1>), dim3((unsigned)tiles),
                       dim3(rs_threads<1>()), 0, s, p);
  else
    hipLaunchKernelGGL((row_sparse_kernel<MODE, 2>), dim3((unsigned)tiles),
                       dim3(rs_threads<2>()), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int row_sparse_dx_split(int64_t n_keep, int in_features, int out_features) {
  const int64_t tiles = (int64_t)(in_features / BT) * ((n_keep + BT - 1) / BT);
  if (tiles == 0 || tiles >= kNumCUs) return 1;
  int64_t split = kNumCUs / tiles;
  const int64_t by_stages = (out_features / BK) / 4;   // >= 4 k-stages per split
  if (split > by_stages) split = by_stages;
  if (split > 8) split = 8;
  return split < 1 ? 1 : (int)split;
}

hipError_t launch_row_sparse_bwd(const RsParams& p, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (p.dx != nullptr) {
    const int64_t threads = p.N * (p.in / 8);
    prof_begin(PKA_KERNEL_RS_ZERO, s);
    hipLaunchKernelGGL(row_sparse_zero_kernel, dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, p);
    prof_end(PKA_KERNEL_RS_ZERO, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.K > 0) {
      prof_begin(PKA_KERNEL_RS_DX, s);
      e = launch_product<kDX>(p, (int64_t)(p.in / BT) * ((p.K + BT - 1) / BT) * p.dx_split, s);
      prof_end(PKA_KERNEL_RS_DX, s);
      if (e != hipSuccess) return e;
      if (p.dx_split > 1) {
        const int64_t threads = p.K * (p.in / 8);
        prof_begin(PKA_KERNEL_RS_DX_REDUCE, s);
        hipLaunchKernelGGL(row_sparse_dx_reduce_kernel, dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, s, p);
        prof_end(PKA_KERNEL_RS_DX_REDUCE, s);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
  }
  if (p.dw != nullptr) {
    prof_begin(PKA_KERNEL_RS_DW, s);
    e = launch_product<kDW>(p, (int64_t)(p.out / BT) * (p.in / BT), s);
    prof_end(PKA_KERNEL_RS_DW, s);
  }
  return e;
}

}  // namespace pka
