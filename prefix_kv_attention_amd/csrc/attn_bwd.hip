// Backward of chunk attention against a frozen prefix cache, gfx950.
//
// Gradient flows through the chunk only: dQ for the chunk's query rows over every
// key they read (cache and chunk), and dK/dV for the chunk's own C keys. The cached
// rows are fixed inputs with no gradient path and receive nothing ("Context-Frozen
// Training", The Gradient Signal; "train: walk the window", Why it's a draft;
// "stop-gradient through context tokens", Known gaps: the attention backward is to
// produce gradient for the kept queries alone).
//
// Kernels, in launch order on the caller's stream (when the dQ row blocks leave CUs
// idle and the chunk dK/dV units fit there, see bwd_dq_kv below, the order is instead:
// bwd_delta, then one grid of dQ row blocks and dK/dV units, then bwd_reduce if the dQ
// rows are split):
//  1. bwd_dq:    delta_i = sum_d dO_id * O_id from the stored bf16 O (prologue; the
//                first split of each row writes it for bwd_dkdv), then per 256
//                packed query rows (GQA packing as in the forward), stream
//                the key tiles: S^T = K Q^T and dP^T = V dO^T (MFMA bf16),
//                P = exp2(S*scale*log2e - LSE*log2e), dS = P (dP - delta) in
//                registers, dQ^T += K^T dS^T with the dS^T registers as the B operand
//                and K^T read from the row-major K tile by the transposing LDS read.
//                Split over key tiles like the forward when the units are too few;
//                fp32 partials are summed by bwd_reduce in a fixed order. MFMA
//                blocks run at raised wave priority (measured ~1.5% faster).
//  2. bwd_dkdv:  per 128 chunk keys of one (window, KV head), stream the packed
//                query rows of all G heads that can see them (token >= key) in tiles
//                of 64: S = Q K^T and dP = dO V^T with keys as MFMA columns, then
//                dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by transposing reads).
//                8 waves, two per SIMD, in two roles over the same 32 keys: one wave
//                holds their K rows in registers and forms S, P and dV, the other
//                holds their V rows and forms dP, dS and dK, taking P from LDS. A
//                staged tile serves all 128 keys (half the query-row re-reads of
//                64-key blocks).
//                The sum over the G heads of a KV head falls out of the packing.
//                When (window, KV head, key block) units are few, each is split
//                over disjoint query-row ranges (a key block gets splits in
//                proportion to the rows that see it) whose fp32 partials
//                bwd_reduce sums in a fixed order (one launch with the dQ sums).
//  Separately, pka_prefix_kv_grad runs the same dK/dV kernel over the last H cache
//  rows of each window (every chunk row sees them), with fp32 outputs.
// No atomics anywhere: every output element is owned by one lane (deterministic).
#include "pka_device.hpp"

namespace pka {
namespace {

constexpr int BN = kKeysPerTile;
constexpr int NW = kWavesPerBlock;
constexpr int NTHR = 64 * NW;

template <int D>
struct DqLds {
  static constexpr int S = D + 8;
  uint16_t k[2][BN * S];
  uint16_t v[2][BN * S];
};

template <int D, int CT>
__device__ __forceinline__ void bwd_dq_body(const BwdParams& p, DqLds<D>& sm, int bid) {
  constexpr int S = DqLds<D>::S;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int ROWS = 32 * NW;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  const int n_rb = p.plan.n_rb, SPL = p.plan.n_split;
  const int L = xcd_logical_id(bid, p.plan.nblk);
  const int rb = L % n_rb;
  const int split = (L / n_rb) % SPL;
  const int grp = L / (n_rb * SPL);
  const int b = grp / p.Hkv, kv = grp % p.Hkv;
  const int G = p.G;
  const int C = (int)p.C;
  const int P = (int)window_prefix(p.plens, b, p.P);  // this window's prefix
  const int rows = G * C;

  const int r = rb * ROWS + wave * 32 + l32;
  const bool row_ok = r < rows;
  const int rr = row_ok ? r : rows - 1;
  const int t = rr / G;
  const int h = kv * G + (rr - t * G);
  const int64_t qrow = ((int64_t)b * p.Hq + h) * C + t;

  const int r_first = rb * ROWS;
  const int r_last = min(rows - 1, r_first + ROWS - 1);
  const int t_min = r_first / G, t_max = r_last / G;
  const int key_end = P + t_max + 1;
  const int n_tiles = (key_end + BN - 1) / BN;
  const int tb = (int)((int64_t)split * n_tiles / SPL);
  const int te = (int)((int64_t)(split + 1) * n_tiles / SPL);

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
  const int64_t bh = (int64_t)b * p.Hkv + kv;
  KVStager<CT, D, NTHR> stg(tid, p.cache, p.kc, p.vc, bh, P, p.C);

  const int k_off = prow(l32) * S + hf * 8;
  const TrOffsets t_off = tr_lane_offsets<S>(lane);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  const int lim = P + t;

  if (tb < te) stg.issue(tb);
  // delta = rowsum(dO * O) of this lane's row: each lane-half holds half of the dO
  // row (the B-operand layout), so read the same half of O and add the halves.
  float dlt;  // computed while the first tile is in flight
  {
    const uint16_t* op = p.o + qrow * D + hf * 8;
    float sdot = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 ov = *reinterpret_cast<const bf16x8*>(op + ks * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) sdot = fmaf((float)ov[e], (float)oreg[ks][e], sdot);
    }
    dlt = pair_sum(sdot);
    // read by bwd_dkdv (which, beside this kernel, reads the delta launch's instead)
    if (split == 0 && row_ok && hf == 0 && !p.plan.dkv_beside) p.delta[qrow] = dlt;
  }

  if (tb < te) {
    stg.store(sm.k[0], sm.v[0]);
    if (tb + 1 < te) stg.issue(tb + 1);
    __syncthreads();
  }
  wait_global_loads();
  f32x16 ndlt;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndlt[i] = -dlt;
  for (int tile = tb; tile < te; ++tile) {
    const int cur = (tile - tb) & 1;
    const uint16_t* kt = sm.k[cur];
    const uint16_t* vt = sm.v[cur];
    const int kbase = tile * BN;
    const bool masked = kbase + BN - 1 > P + t_min;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // dP^T starts from -delta (this lane's row), so the chain yields dP - delta.
      f32x16 st = f32x16{}, dpt = ndlt;
      __builtin_amdgcn_s_setprio(1);
      {
        bf16x8 a[NKS][2];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int off = k_off + kb * 32 * S + ks * 16;
          a[ks][0] = *reinterpret_cast<const bf16x8*>(&kt[off]);
          a[ks][1] = *reinterpret_cast<const bf16x8*>(&vt[off]);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          st = mfma32(a[ks][0], qreg[ks], st);
          dpt = mfma32(a[ks][1], oreg[ks], dpt);
        }
        sched_ahead<2 * NKS, kDqReadAheadSP, 1>();
      }
      __builtin_amdgcn_s_setprio(0);
      if (masked) {
        const int rel = lim - kbase - hf * 4;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + (i >> 2) * 8 + (i & 3) > rel) st[i] = -INFINITY;
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(st[i], c, -lse2));
        dsb[i >> 3][i & 7] = (__bf16)(pv * dpt[i]);
      }
      __builtin_amdgcn_s_setprio(1);
      {
        bf16x8 a[2][NDB];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int db = 0; db < NDB; ++db) a[s][db] = lds_tr_operand<S>(kt, t_off, kb * 32 + s * 16, db * 32);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[db] = mfma32(a[s][db], dsb[s], acc[db]);
        sched_ahead<2 * NDB, kDqReadAheadDQ, 2>();
      }
      __builtin_amdgcn_s_setprio(0);
    }

    if (tile + 1 < te) {
      stg.store(sm.k[cur ^ 1], sm.v[cur ^ 1]);
      if (tile + 2 < te) stg.issue(tile + 2);
      __syncthreads();
    }
  }

  if (!row_ok) return;
  const float sc = p.scale;
  if (SPL == 1) {
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

template <int D, int CT>
__global__ __launch_bounds__(NTHR) void bwd_dq_kernel(BwdParams p) {
  __shared__ __align__(16) DqLds<D> sm;
  bwd_dq_body<D, CT>(p, sm, (int)blockIdx.x);
}

// ------------------------------------------------------------------ dK / dV
constexpr int BQ = 64;                      // packed query rows per step
constexpr int KB = kDkvKeysPerBlock;        // keys per dK/dV workgroup (128)

template <int D>
struct DkvLds {
  static constexpr int S = D + 8;
  uint16_t q[2][BQ * S];
  uint16_t g[2][BQ * S];   // dO
  // P of the step (fp32), handed from the S / P / dV waves to the dP / dS / dK waves of
  // the same keys: [key block][row half][group of 4 result registers][lane][4].
  __align__(16) float pt[4][2][4][64 * 4];
  __align__(16) float lse2[2][BQ];
  __align__(16) float dlt[2][BQ];   // -delta of the staged rows
  __align__(16) int tok[2][BQ];
};

constexpr int NTHR_KV = 512;   // 8 waves: two roles x 4 key blocks of 32

// dK/dV of one block of 128 keys of one (window, KV head), over the packed query
// rows of all G heads that see them. PREFIX = false: the chunk's own keys (causal:
// rows whose token is >= the key), bf16 outputs dk, dv [B][Hkv][C][D].
// PREFIX = true: the last `horizon` cache rows [P_b - H, P_b) of the window (every
// chunk row sees them), dequantised on load like the forward; fp32 outputs
// dkp, dvp [B][Hkv][H][D] whose row h is cache row P_b - H + h (zero when that row
// does not exist because P_b < H).
// Waves kw = 0..3 and 4 + kw own keys kw*32 .. kw*32+31 over both 32-row halves of
// every step of 64 rows, in two roles. Wave kw holds the keys' K rows in registers
// (the B operand of S = Q K^T), forms P = exp2(S * scale * log2 e - LSE * log2 e) with
// the causal mask, hands P to LDS in fp32 and adds dV^T += dO^T P. Wave 4 + kw (the
// other wave of the same SIMD) holds the keys' V rows, forms dP - delta = dO V^T -
// delta, and after the hand-over dS = P (dP - delta) and dK^T += Q^T dS. So every MFMA
// reads one operand from LDS, each output element has one owner (no reduction across
// waves), and the first role's softmax runs while the second role's MFMAs issue. The
// next step's rows are staged where each role would otherwise wait: the dO rows by the
// second role after its dP chain, the Q rows by the first role after its dV chain, the
// LSE / delta by wave 0 after its softmax. Two barriers per step: P is written, and the
// step's tiles are free again. The S and dP chains read all their LDS operands before
// their first MFMA (left to the compiler, the reads ran two MFMAs ahead and each pair of
// MFMAs waited out one read).
template <int D, int CT, bool PREFIX, bool BESIDE>
__device__ __forceinline__ void bwd_kv_body(const BwdParams& p, DkvLds<D>& sm, int bid,
                                            int nblk) {
  constexpr int S = DkvLds<D>::S;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CH = D / 8;
  constexpr int NRT = NTHR_KV / 2;            // threads of one role
  constexpr int RT = BQ * CH / NRT;           // rows a thread stages per step (4 or 2)
  static_assert(KB == 32 * 4, "four key blocks of 32");
  static_assert(RT * NRT == BQ * CH, "one staging task per thread of a role");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int kw = wave & 3;           // key block of this wave
  const bool second = wave >= 4;     // dP / dS / dK role
  const int C = (int)p.C;
  const int G = p.G;
  const int rows = G * C;
  const int NK = PREFIX ? (int)p.horizon : C;   // keys of this launch per (b, kv)
  const int nkb = (NK + KB - 1) / KB;
  const int RS = p.plan.n_dkv_split;   // > 1: partials for bwd_reduce
  // Neighbouring logical ids (key blocks of one unit) share an XCD and so read the
  // unit's Q / dO rows from that XCD's L2.
  // Beside the dQ row blocks, unit j goes to XCD j % 8 as launched: every XCD gets
  // units of every size, and (with a multiple of 8 (window, KV head) pairs) all units of
  // one pair share an XCD.
  const int L = BESIDE ? bid : xcd_logical_id(bid, nblk);
  int rsplit, kblk, grp, RSk;   // RSk: row splits of this key block
  if constexpr (BESIDE) {
    // beside the dQ row blocks: one unit per key block, largest (block 0) first
    const int groups = p.B * p.Hkv;
    kblk = L / groups;
    grp = L - kblk * groups;
    rsplit = 0;
    RSk = 1;
  } else if (!PREFIX && p.plan.dkv_nkb > 0) {
    const int per = p.plan.dkv_first[nkb];
    grp = L / per;
    const int r = L - grp * per;
    kblk = 0;
    while (kblk + 1 < nkb && p.plan.dkv_first[kblk + 1] <= r) ++kblk;
    rsplit = r - p.plan.dkv_first[kblk];
    RSk = p.plan.dkv_first[kblk + 1] - p.plan.dkv_first[kblk];
  } else {
    rsplit = L % RS;
    kblk = (L / RS) % nkb;
    grp = L / (RS * nkb);
    RSk = RS;
  }
  const int b = grp / p.Hkv, kv = grp % p.Hkv;
  const int64_t bh = (int64_t)b * p.Hkv + kv;
  const int key = kblk * KB + kw * 32 + l32;  // key index of this launch (output row)
  const int64_t Pb = PREFIX ? window_prefix(p.plens, b, p.P) : 0;
  // A prefix row that does not exist (P_b < H) contributes and gets exactly zero.
  const bool key_ok = key < NK && (!PREFIX || Pb - NK + key >= 0);

  // This wave's fixed MFMA operand: the K (first role) or V (second role) row of key
  // `key`, converted to bf16, as the B operand of S or dP: k-step ks of lane (l32, hf)
  // is values ks*16 + hf*8 .. +7. Missing keys are zero rows.
  bf16x8 kvop[NKS];
  {
    constexpr int ESZ = (CT == kQ8) ? 1 : 2;
    const char* base = static_cast<const char*>(second ? p.cache.v : p.cache.k) +
                       bh * p.cache.cap * D * ESZ;
    const uint16_t* scl =
        (CT == kQ8) ? (second ? p.cache.vs : p.cache.ks) + bh * p.cache.cap * (D / 32) : nullptr;
    const uint16_t* crow = (second ? p.vc : p.kc) + (bh * C + key) * D;
    const int64_t j = Pb - NK + key;   // cache row of a prefix key
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int d0 = ks * 16 + hf * 8;
      u32x4 w = u32x4{0u, 0u, 0u, 0u};
      if constexpr (PREFIX) {
        if (key_ok) {
          RawRow8 r;
          load_row8<CT, D>(r, base, scl, nullptr, Pb, 0, j, d0);
          w = to_bf16x8<CT>(r, true);
        }
      } else {
        if (key < NK) w = *reinterpret_cast<const u32x4*>(crow + d0);
      }
      kvop[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const float c = p.scale_log2;

  // Rows whose token is >= the block's first key can see some key of it.
  const int r_unit = PREFIX ? 0 : kblk * KB * G;
  const int steps_unit = (rows - r_unit + BQ - 1) / BQ;
  const int s_lo = (int)((int64_t)rsplit * steps_unit / RSk);
  const int s_hi = (int)((int64_t)(rsplit + 1) * steps_unit / RSk);
  const int r_begin = r_unit + s_lo * BQ;   // this split's rows
  const int n_steps = s_hi - s_lo;
  // Packed rows from clean_from on have tokens >= the block's last key: no mask.
  const int clean_from = (kblk * KB + KB - 1) * G;
  // Packed row rr is token rr / G of query head kv*G + rr % G, at row offset
  // (rr % G) * C + rr / G from the first row of that head. Each thread follows its rows
  // from step to step (+BQ packed rows) without dividing.
  const int dt_step = BQ / G, dg_step = BQ % G;
  const int64_t head0 = (int64_t)b * p.Hq + kv * G;   // first query head of this KV head
  const int ro_step = dg_step * C + dt_step;           // row offset change per step
  const int ro_wrap = 1 - G * C;                       // ... plus this when g wraps
  auto advance = [&](int& ro, int& g) {
    ro += ro_step;
    g += dg_step;
    if (g >= G) {
      g -= G;
      ro += ro_wrap;
    }
  };
  auto start = [&](int rr, int& ro, int& g) {
    const int t = rr / G;
    g = rr - t * G;
    ro = g * C + t;
  };
  // Row staging: the first role moves the Q rows of a step, the second the dO rows,
  // each thread RT rows of 8 values, loaded a step ahead of the LDS write. The rows of
  // the G query heads of this KV head are one block of G * C rows (under 4 GiB, checked
  // by the host); buffer loads address it with 32-bit byte offsets, and an offset past
  // its end (a padding row of the last step) reads zero instead of faulting.
  const int ts = tid & (NRT - 1);
  const int tr0 = (ts / CH) * RT, td0 = (ts % CH) * 8;
  const __amdgpu_buffer_rsrc_t rows_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>((second ? p.d_o : p.q) + head0 * C * D), 0,
      (int)((uint32_t)G * (uint32_t)C * (uint32_t)(D * 2)), 0x00020000);
  uint16_t* const dst0 = second ? sm.g[0] : sm.q[0];
  uint32_t rb[RT];   // byte offset of each staged row's 8 values in the block
  int gq[RT];        // head in the group of each staged row
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    int ro;
    start(r_begin + tr0 + i, ro, gq[i]);
    rb[i] = (uint32_t)ro * (D * 2) + td0 * 2;
  }
  const uint32_t rb_step = (uint32_t)ro_step * (D * 2);
  const uint32_t rb_wrap = (uint32_t)ro_wrap * (D * 2);   // modulo 2^32
  u32x4 rq[RT];
  int rows_left = 0;   // rows of the issued step that exist (>= BQ: all)
  auto issue = [&](int step) {   // called for steps 0, 1, 2, ... in order
    rows_left = rows - (r_begin + step * BQ);
#pragma unroll
    for (int i = 0; i < RT; ++i)
      rq[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rows_rsrc, (int)rb[i], 0, 0));
    if (dg_step == 0) {   // G divides BQ: every row moves BQ / G tokens
#pragma unroll
      for (int i = 0; i < RT; ++i) rb[i] += rb_step;
    } else {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        gq[i] += dg_step;
        const bool wrap = gq[i] >= G;
        gq[i] -= wrap ? G : 0;
        rb[i] += rb_step + (wrap ? rb_wrap : 0u);
      }
    }
  };
  auto stage = [&](int buf) {
    if (rows_left < BQ) {   // the last step: zero the rows past the end
#pragma unroll
      for (int i = 0; i < RT; ++i)
        if (tr0 + i >= rows_left) rq[i] = u32x4{0u, 0u, 0u, 0u};
    }
    uint16_t* dst = dst0 + buf * (BQ * S);
#pragma unroll
    for (int i = 0; i < RT; ++i)
      *reinterpret_cast<u32x4*>(&dst[prow(tr0 + i) * S + td0]) = rq[i];
  };
  if (n_steps > 0) {
    issue(0);
    stage(0);
    if (n_steps > 1) issue(1);
  }

  float* ptw = &sm.pt[kw][0][0][lane * 4];   // this key block's P, lane's 4 values
  const int a_off = prow(l32) * S + hf * 8;  // operand rows of row half 0 of a step
  const TrOffsets t_off = tr_lane_offsets<S>(lane);

  if (!second) {
    // Wave 0 stages the LSE, -delta and token of every row of a step (one row per
    // lane), loads a step ahead of the LDS write.
    const float* lse_head = p.lse + head0 * C;
    const float* dlt_head = p.delta + head0 * C;
    int rol = 0, gl = 0;
    start(r_begin + lane, rol, gl);
    float pl = 0.f, pd = 0.f;   // raw LSE and delta: scaled when written to LDS
    int ptok = -1;
    auto issue_l = [&](int step) {
      // Unconditional loads (a padding row reads the first row of the head): any use
      // of a loaded value here would wait for the load.
      const bool valid = r_begin + step * BQ + lane < rows;
      const int off = valid ? rol : 0;
      pl = lse_head[off];
      pd = dlt_head[off];
      ptok = valid ? (rol - gl * C) : -1;
      advance(rol, gl);
    };
    auto stage_l = [&](int buf) {
      const bool valid = ptok >= 0;
      sm.lse2[buf][lane] = valid ? pl * kLog2e : 0.f;
      sm.dlt[buf][lane] = valid ? -pd : 0.f;   // negated: the dP chain starts from it
      sm.tok[buf][lane] = ptok;
    };
    if (wave == 0 && n_steps > 0) {
      issue_l(0);
      stage_l(0);
      if (n_steps > 1) issue_l(1);
    }
    f32x16 accv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) accv[db] = f32x16{};
    __syncthreads();   // step 0's rows are in LDS
    // One wait for the fixed operand (and wave 0's first LSE / delta loads): otherwise
    // the compiler waits for every load at the loop top, the next steps' ones included.
    wait_global_loads();
    for (int step = 0; step < n_steps; ++step) {
      const int cur = step & 1;
      const uint16_t* qt = sm.q[cur];
      const uint16_t* gt = sm.g[cur];
      const bool diag = !PREFIX && r_begin + step * BQ < clean_from;
      // S of this wave's 32 keys over both row halves. Register i of a result is row
      // (i / 4) * 8 + hf * 4 + i % 4 of the half, key l32.
      f32x16 sv[2] = {f32x16{}, f32x16{}};
      bf16x8 opa[2][NKS];
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          opa[rh][ks] = *reinterpret_cast<const bf16x8*>(&qt[a_off + rh * 32 * S + ks * 16]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          sv[rh] = mfma32(opa[rh][ks], kvop[ks], sv[rh]);
      bf16x8 pb[2][2];
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int q0 = rh * 32 + g4 * 8 + hf * 4;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[cur][q0]);
          const int4 t4 = *reinterpret_cast<const int4*>(&sm.tok[cur][q0]);
          const int tk[4] = {t4.x, t4.y, t4.z, t4.w};
          f32x4 pf;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int i = g4 * 4 + jj;
            const float e = __builtin_amdgcn_exp2f(fmaf(sv[rh][i], c, -l4[jj]));
            // Prefix keys are seen by every row; padding rows past the last one have
            // zero q and dO and so add nothing. Chunk keys: causal, checked only in
            // the steps that reach below the block's last key.
            const float pv = (!PREFIX && diag && key > tk[jj]) ? 0.f : e;
            pf[jj] = pv;
            pb[rh][i >> 3][i & 7] = (__bf16)pv;
          }
          *reinterpret_cast<f32x4*>(ptw + (rh * 4 + g4) * 256) = pf;
        }
      // The next step's LSE / delta go to the other buffer, read last in the previous step.
      if (wave == 0 && step + 1 < n_steps) {
        stage_l(cur ^ 1);
        if (step + 2 < n_steps) issue_l(step + 2);
      }
      __syncthreads();   // P is in LDS
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int ss = 0; ss < 2; ++ss)
            accv[db] = mfma32(lds_tr_operand<S>(gt, t_off, rh * 32 + ss * 16, db * 32),
                              pb[rh][ss], accv[db]);
      // The next step's Q rows go to the other buffer, read last in the previous step.
      if (step + 1 < n_steps) {
        stage(cur ^ 1);
        if (step + 2 < n_steps) issue(step + 2);
      }
      __syncthreads();   // this step's tiles and P are free
    }
    if (key >= NK) return;
    if (PREFIX && RS == 1) {
      float* pv = p.dvp + (bh * NK + key) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + g4 * 8 + hf * 4;
          *reinterpret_cast<f32x4*>(pv + d) =
              key_ok ? f32x4{accv[db][g4 * 4 + 0], accv[db][g4 * 4 + 1], accv[db][g4 * 4 + 2],
                             accv[db][g4 * 4 + 3]}
                     : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      return;
    }
    if (RS > 1) {
      // fp32 partials of this row split, summed in split order by bwd_reduce.
      const int64_t nkey = (int64_t)p.B * p.Hkv * NK;
      float* pv = p.ws_dkv + ((int64_t)rsplit * 2 * nkey + nkey + bh * NK + key) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + g4 * 8 + hf * 4;
          *reinterpret_cast<f32x4*>(pv + d) =
              key_ok ? f32x4{accv[db][g4 * 4 + 0], accv[db][g4 * 4 + 1], accv[db][g4 * 4 + 2],
                             accv[db][g4 * 4 + 3]}
                     : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      return;
    }
    uint16_t* dvp = p.dv + (bh * C + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hf * 4;
        u32x2 wv;
        wv.x = pack_bf16(accv[db][g4 * 4 + 0], accv[db][g4 * 4 + 1]);
        wv.y = pack_bf16(accv[db][g4 * 4 + 2], accv[db][g4 * 4 + 3]);
        *reinterpret_cast<u32x2*>(dvp + d) = wv;
      }
    return;
  }

  // ---- second role: dP, dS, dK
  f32x16 acck[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acck[db] = f32x16{};
  __syncthreads();   // step 0's rows are in LDS
  // One wait for every load so far (the fixed operand, step 1's rows): otherwise the
  // compiler waits at the loop top on each iteration, and that wait also covers the
  // rows just requested for two steps ahead.
  wait_global_loads();
  for (int step = 0; step < n_steps; ++step) {
    const int cur = step & 1;
    const uint16_t* qt = sm.q[cur];
    const uint16_t* gt = sm.g[cur];
    // dP of this wave's keys over both row halves; the chain starts from -delta of
    // its rows, so it yields dP - delta (register layout as S).
    f32x16 dp[2];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dlt[cur][rh * 32 + g4 * 8 + hf * 4]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dp[rh][g4 * 4 + jj] = d4[jj];
      }
    bf16x8 opa[2][NKS];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        opa[rh][ks] = *reinterpret_cast<const bf16x8*>(&gt[a_off + rh * 32 * S + ks * 16]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rh = 0; rh < 2; ++rh)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        dp[rh] = mfma32(opa[rh][ks], kvop[ks], dp[rh]);
    // The next step's dO rows go to the other buffer, read last in the previous step.
    if (step + 1 < n_steps) {
      stage(cur ^ 1);
      if (step + 2 < n_steps) issue(step + 2);
    }
    __syncthreads();   // P is in LDS
    bf16x8 dsb[2][2];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 pf = *reinterpret_cast<const f32x4*>(ptw + (rh * 4 + g4) * 256);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int i = g4 * 4 + jj;
          dsb[rh][i >> 3][i & 7] = (__bf16)(pf[jj] * dp[rh][i]);
        }
      }
#pragma unroll
    for (int rh = 0; rh < 2; ++rh)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss)
          acck[db] = mfma32(lds_tr_operand<S>(qt, t_off, rh * 32 + ss * 16, db * 32),
                            dsb[rh][ss], acck[db]);
    __syncthreads();   // this step's tiles and P are free
  }
  if (key >= NK) return;
  const float sc = p.scale;
  if (PREFIX && RS == 1) {
    float* pk = p.dkp + (bh * NK + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hf * 4;
        *reinterpret_cast<f32x4*>(pk + d) =
            key_ok ? f32x4{acck[db][g4 * 4 + 0] * sc, acck[db][g4 * 4 + 1] * sc,
                           acck[db][g4 * 4 + 2] * sc, acck[db][g4 * 4 + 3] * sc}
                   : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    return;
  }
  if (RS > 1) {
    const int64_t nkey = (int64_t)p.B * p.Hkv * NK;
    float* pk = p.ws_dkv + ((int64_t)rsplit * 2 * nkey + bh * NK + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hf * 4;
        *reinterpret_cast<f32x4*>(pk + d) =
            key_ok ? f32x4{acck[db][g4 * 4 + 0] * sc, acck[db][g4 * 4 + 1] * sc,
                           acck[db][g4 * 4 + 2] * sc, acck[db][g4 * 4 + 3] * sc}
                   : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    return;
  }
  uint16_t* dkp = p.dk + (bh * C + key) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + g4 * 8 + hf * 4;
      u32x2 wk;
      wk.x = pack_bf16(acck[db][g4 * 4 + 0] * sc, acck[db][g4 * 4 + 1] * sc);
      wk.y = pack_bf16(acck[db][g4 * 4 + 2] * sc, acck[db][g4 * 4 + 3] * sc);
      *reinterpret_cast<u32x2*>(dkp + d) = wk;
    }
}

template <int D, int CT, bool PREFIX>
__global__ __launch_bounds__(NTHR_KV) void bwd_kv_kernel(BwdParams p) {
  __shared__ __align__(16) DkvLds<D> sm;
  bwd_kv_body<D, CT, PREFIX, false>(p, sm, (int)blockIdx.x, (int)gridDim.x);
}

// The chunk backward in one grid when the dQ row blocks leave CUs idle: workgroups
// [0, nblk) are the dQ row blocks, the rest the chunk dK/dV units (one per key block).
// The hardware starts workgroups in index order, so the units take the idle CUs while
// the dQ blocks run. The plan takes this grid only when every unit has an idle CU from
// the start and should end within the dQ blocks' time: a unit left waiting was not
// placed on a CU that an earlier unit freed, only on one a dQ block freed.
template <int D, int CT>
__global__ __launch_bounds__(NTHR) void bwd_dq_kv_kernel(BwdParams p) {
  static_assert(NTHR == NTHR_KV, "one block size for both");
  __shared__ __align__(16) union {
    DqLds<D> dq;
    DkvLds<D> kv;
  } sm;
  const int bid = (int)blockIdx.x;
  if (bid < p.plan.nblk)
    bwd_dq_body<D, CT>(p, sm.dq, bid);
  else
    bwd_kv_body<D, kBF16, false, true>(p, sm.kv, bid - p.plan.nblk,
                                       (int)gridDim.x - p.plan.nblk);
}

// delta_i = sum_d dO_id * O_id (fp32) of every chunk row, for the dK/dV units that run
// beside the dQ row blocks: CH = D / 8 consecutive lanes share a row, 8 values each.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  constexpr int CH = D / 8;
  const int64_t nrow = (int64_t)p.B * p.Hq * p.C;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / CH;
  const int c8 = (int)(idx % CH);
  const bool ok = row < nrow;   // every lane takes part in the lane sums below
  const int64_t r = ok ? row : 0;
  const u32x4 g = *reinterpret_cast<const u32x4*>(p.d_o + r * D + c8 * 8);
  const u32x4 o = *reinterpret_cast<const u32x4*>(p.o + r * D + c8 * 8);
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // element copies first: a bit_cast of a subscripted vector element reads element 0
    const uint32_t gw = g[e], ow = o[e];
    dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, gw),
                                          __builtin_bit_cast(bf16x2, ow), dot, false);
  }
  dot += dpp_f32<0xB1>(dot);    // quad_perm [1, 0, 3, 2]
  dot += dpp_f32<0x4E>(dot);    // quad_perm [2, 3, 0, 1]
  dot += dpp_f32<0x141>(dot);   // row_half_mirror: the sum of 8 lanes
  if constexpr (CH == 16) dot += dpp_f32<0x140>(dot);   // row_mirror: of 16
  if (ok && c8 == 0) p.delta[row] = dot;
}

// Sums of split partials, in split order, written as bf16 (one launch for both):
// threads [0, n_dq) reduce dQ rows (prefix split of the dQ kernel), the rest reduce
// dK and dV rows (query-row split of the dK/dV kernel).
template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p, int64_t n_dq,
                                                         int64_t n_dkv, int64_t nk) {
  constexpr int CH = D / 8;
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float* src;
  int64_t stride;  // floats between consecutive splits
  int nsplit;
  uint16_t* dst = nullptr;
  float* dst32 = nullptr;
  if (idx < n_dq) {
    const int64_t nrow = (int64_t)p.B * p.Hq * p.C;
    const int64_t row = idx / CH;
    const int c8 = (int)(idx % CH);
    src = p.ws_dq + row * D + c8 * 8;
    stride = nrow * D;
    nsplit = p.plan.n_split;
    dst = p.dq + row * D + c8 * 8;
  } else {
    idx -= n_dq;
    if (idx >= n_dkv) return;   // n_dkv is 0 when dK/dV rows were not split
    const int64_t nkey = (int64_t)p.B * p.Hkv * nk;
    const int which = (int)(idx / (nkey * CH));   // 0: dK, 1: dV
    const int64_t rem = idx - which * nkey * CH;
    const int64_t row = rem / CH;
    const int c8 = (int)(rem % CH);
    src = p.ws_dkv + (which * nkey + row) * D + c8 * 8;
    stride = 2 * nkey * D;
    nsplit = p.plan.n_dkv_split;
    if (!F32OUT && p.plan.dkv_nkb > 0) {   // chunk keys: splits of the row's key block
      const int kb = (int)((row % nk) / KB);
      nsplit = p.plan.dkv_first[kb + 1] - p.plan.dkv_first[kb];
    }
    if (F32OUT)
      dst32 = (which ? p.dvp : p.dkp) + row * D + c8 * 8;
    else
      dst = (which ? p.dv : p.dk) + row * D + c8 * 8;
  }
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const f32x4* v = reinterpret_cast<const f32x4*>(src + (int64_t)s * stride);
    const f32x4 a = v[0], bq = v[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] += a[i];
      o[4 + i] += bq[i];
    }
  }
  if (F32OUT) {
    reinterpret_cast<f32x4*>(dst32)[0] = f32x4{o[0], o[1], o[2], o[3]};
    reinterpret_cast<f32x4*>(dst32)[1] = f32x4{o[4], o[5], o[6], o[7]};
  } else {
    *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]),
                                           pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7])};
  }
}

template <int D, int CT>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
  const int64_t nrow = (int64_t)p.B * p.Hq * p.C;
  hipError_t e;
  if (p.plan.dkv_beside) {
    const int64_t units = (int64_t)p.B * p.Hkv * ((p.C + KB - 1) / KB);
    prof_begin(PKA_KERNEL_BWD_PREP, s);
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((nrow * (D / 8) + 255) / 256)),
                       dim3(256), 0, s, p);
    prof_end(PKA_KERNEL_BWD_PREP, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    prof_begin(PKA_KERNEL_BWD_DQ, s);
    hipLaunchKernelGGL((bwd_dq_kv_kernel<D, CT>), dim3((unsigned)(p.plan.nblk + units)),
                       dim3(NTHR), 0, s, p);
    prof_end(PKA_KERNEL_BWD_DQ, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.plan.n_split > 1) {
      const int64_t n_dq = nrow * (D / 8);
      prof_begin(PKA_KERNEL_BWD_DQ_REDUCE, s);
      hipLaunchKernelGGL((bwd_reduce_kernel<D, false>), dim3((unsigned)((n_dq + 255) / 256)),
                         dim3(256), 0, s, p, n_dq, (int64_t)0, p.C);
      prof_end(PKA_KERNEL_BWD_DQ_REDUCE, s);
      e = hipGetLastError();
    }
    return e;
  }
  prof_begin(PKA_KERNEL_BWD_DQ, s);
  hipLaunchKernelGGL((bwd_dq_kernel<D, CT>), dim3(p.plan.nblk), dim3(NTHR), 0, s, p);
  prof_end(PKA_KERNEL_BWD_DQ, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const int nkb = (int)((p.C + KB - 1) / KB);
  const int per_grp = p.plan.dkv_nkb > 0 ? p.plan.dkv_first[nkb] : nkb * p.plan.n_dkv_split;
  prof_begin(PKA_KERNEL_BWD_DKDV, s);
  hipLaunchKernelGGL((bwd_kv_kernel<D, kBF16, false>), dim3(p.B * p.Hkv * per_grp),
                     dim3(NTHR_KV), 0, s, p);
  prof_end(PKA_KERNEL_BWD_DKDV, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const int64_t n_dq = p.plan.n_split > 1 ? nrow * (D / 8) : 0;
  const int64_t n_dkv = p.plan.n_dkv_split > 1 ? 2 * (int64_t)p.B * p.Hkv * p.C * (D / 8) : 0;
  if (n_dq + n_dkv > 0) {
    prof_begin(PKA_KERNEL_BWD_DQ_REDUCE, s);
    hipLaunchKernelGGL((bwd_reduce_kernel<D, false>),
                       dim3((unsigned)((n_dq + n_dkv + 255) / 256)), dim3(256), 0, s, p, n_dq,
                       n_dkv, p.C);
    prof_end(PKA_KERNEL_BWD_DQ_REDUCE, s);
    e = hipGetLastError();
  }
  return e;
}

template <int D, int CT>
hipError_t launch_prefix_kv_t(const BwdParams& p, hipStream_t s) {
  hipError_t e;
  const int nkb = (int)((p.horizon + KB - 1) / KB);
  prof_begin(PKA_KERNEL_PREFIX_KV, s);
  hipLaunchKernelGGL((bwd_kv_kernel<D, CT, true>),
                     dim3(p.B * p.Hkv * nkb * p.plan.n_dkv_split), dim3(NTHR_KV), 0, s, p);
  prof_end(PKA_KERNEL_PREFIX_KV, s);
  if ((e = hipGetLastError()) != hipSuccess || p.plan.n_dkv_split == 1) return e;
  const int64_t n_dkv = 2 * (int64_t)p.B * p.Hkv * p.horizon * (D / 8);
  prof_begin(PKA_KERNEL_PREFIX_KV_REDUCE, s);
  hipLaunchKernelGGL((bwd_reduce_kernel<D, true>), dim3((unsigned)((n_dkv + 255) / 256)),
                     dim3(256), 0, s, p, (int64_t)0, n_dkv, p.horizon);
  prof_end(PKA_KERNEL_PREFIX_KV_REDUCE, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefix_kv(const BwdParams& p, int D, int cache_type, hipStream_t s) {
  if (D == 128) {
    if (cache_type == kF16) return launch_prefix_kv_t<128, kF16>(p, s);
    if (cache_type == kBF16) return launch_prefix_kv_t<128, kBF16>(p, s);
    return launch_prefix_kv_t<128, kQ8>(p, s);
  }
  if (cache_type == kF16) return launch_prefix_kv_t<64, kF16>(p, s);
  if (cache_type == kBF16) return launch_prefix_kv_t<64, kBF16>(p, s);
  return launch_prefix_kv_t<64, kQ8>(p, s);
}

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
