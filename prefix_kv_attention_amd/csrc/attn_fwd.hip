// Forward of chunk attention against a frozen prefix cache, gfx950.
//
// Computes, for every chunk query row, softmax attention over the cached context
// rows 0..P-1 plus the chunk's own keys 0..i, writing O and the natural-log LSE
// ("Context-Frozen Training", The Solution, Phase 2: the decision tokens run
// against the frozen KV cache; "train: walk the window", What it is: each chunk
// reads the cached prefix as constants).
//
// Design (MI355X):
//  * GQA packing: one workgroup of 8 waves serves 256 packed rows of one (window,
//    KV head); packed row r is token r / G of query head kv*G + r % G, so every
//    query head that shares a KV head reads each staged K/V tile from LDS.
//  * Each wave owns 32 rows. Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16, so lane l holds the scores of query row l % 32: the
//    row max / row sum need one exchange (lane l <-> l^32) per tile, and the running
//    max, sum and rescale factor are per-lane scalars.
//  * O^T += V^T P^T: the S^T registers (converted to bf16) are the B operand as is;
//    the V^T operand is read from the row-major V tile with the transposing LDS
//    read, so no transposed copy is ever staged.
//  * Ping-pong of the two waves of each SIMD (bf16 caches, fwd_kernel): waves 0-3 and
//    4-7 run the same sequence of phases, one phase apart, with a workgroup barrier
//    between phases. A phase of one wave is either its MFMA block (S of tile i, P V of
//    tile i - 1) or its VALU block (the online softmax of tile i, and staging). So
//    while one wave of a SIMD keeps the matrix core busy, the other's exp2 / fma / pack
//    work runs beside it instead of after it (measured with a register-only model of
//    the tile: 2,100 cycles per tile against 2,066 for the MFMAs alone and 2,593 when
//    each wave runs its MFMAs and its VALU work back to back). F16 and q8_0 caches take
//    fwd_serial_kernel instead, where each wave runs both blocks itself and the tile
//    staging (with its conversion to bf16) is spread over all eight waves: there the
//    staging makes the VALU phase longer than the MFMA phase, and the ping-pong was
//    measured slower (q8_0 at P = 63488: 0.710 ms against 0.662 ms).
//  * The key sequence [cache rows ; chunk rows] is streamed in 64-key tiles through
//    two LDS buffers per tensor; waves 0-3 stage the K tiles and waves 4-7 the V tiles,
//    each in its own VALU phase, loading one phase pair ahead. Tiles that lie wholly
//    in the cache use a fast path (uniform base pointer, fixed per-thread offsets);
//    F16 / q8_0 rows are converted to bf16 while staging (dequantised on load). Only
//    tiles that cross the causal diagonal are masked.
//  * The probabilities of a tile are taken against the running reference max; the
//    reference is raised to the exact row max (and the accumulator rescaled) only
//    when it is unset or a lane's partial row sum of the tile exceeds 2^8, which any
//    probability above 2^8 forces. So the max reduction and the rescale are skipped
//    on almost every tile, and probabilities stay <= 2^8, which bf16 and fp32 hold
//    exactly enough. The result is the same softmax (any reference max gives it).
//  * LDS operand reads run several MFMAs ahead of their use (sched_chain2): without
//    that the wave waits out the LDS latency at each MFMA.
//  * With FwdParams::append the same launch writes the chunk's K/V into the cache
//    rows [P_b, P_b + C) after its last tile (the re-decode into the cache).
//  * When (window, KV head, row block) units are too few to fill 256 CUs, the key
//    tiles are split over several workgroups; partial (O, LSE) are merged by
//    fwd_combine in a fixed order (deterministic).
//  * Workgroups are renumbered so each XCD works on a contiguous range of units and
//    the K/V tiles they share stay in that XCD's L2.
#include "pka_device.hpp"

namespace pka {
namespace {

constexpr int BN = kKeysPerTile;   // keys per tile
constexpr int NW = kWavesPerBlock; // waves per workgroup
constexpr int NTHR = 64 * NW;
// Largest probability a tile may produce before the reference max is raised: 2^8
// (bf16 bits 0x4380); any larger value is exact enough in bf16 and fp32 but could, if
// left unchecked, grow past what the sums hold.
constexpr uint16_t kProbLimitBits = 0x4380;
constexpr float kSumLimit = 256.f;  // bound on a lane's partial row sum of one tile
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <int D>
struct FwdLds {
  static constexpr int S = D + 8;
  uint16_t k[2][BN * S];
  uint16_t v[2][BN * S];
};

template <int D, int CT>
__global__ __launch_bounds__(NTHR) void fwd_kernel(FwdParams p) {
  __shared__ __align__(16) FwdLds<D> sm;
  constexpr int S = FwdLds<D>::S;
  constexpr int NKS = D / 16;   // k-steps over head_dim
  constexpr int NDB = D / 32;   // 32-row blocks of O^T

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  const int n_rb = p.plan.n_rb, SPL = p.plan.n_split;
  const int L = xcd_logical_id(blockIdx.x, p.plan.nblk);
  const int rb = L % n_rb;
  const int split = (L / n_rb) % SPL;
  const int grp = L / (n_rb * SPL);
  const int b = grp / p.Hkv, kv = grp % p.Hkv;
  const int G = p.G;
  const int C = (int)p.C;
  const int P = (int)window_prefix(p.plens, b, p.P);  // this window's prefix
  const int rows = G * C;
  constexpr int ROWS = 32 * NW;

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

  bf16x8 qreg[NKS];
  {
    const uint16_t* qp = p.q + qrow * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qreg[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }

  // Ping-pong: waves 0-3 (group 0, one per SIMD) and waves 4-7 (group 1) run the same
  // phases one phase apart, so on every SIMD one wave issues its MFMA block while the
  // other runs its softmax VALU and staging; a barrier ends every phase. Group 0
  // stages the K tiles, group 1 the V tiles.
  const int grp_w = __builtin_amdgcn_readfirstlane(wave) >> 2;
  const int64_t bh = (int64_t)b * p.Hkv + kv;
  TileStager<CT, D, NTHR / 2, 2> stg(tid & (NTHR / 2 - 1), grp_w ? p.cache.v : p.cache.k,
                                     grp_w ? p.cache.vs : p.cache.ks, grp_w ? p.vc : p.kc, bh,
                                     p.cache.cap, P, p.C);
  uint16_t* const own0 = grp_w ? sm.v[0] : sm.k[0];
  uint16_t* const own1 = grp_w ? sm.v[1] : sm.k[1];

  // Per-lane LDS offsets of the MFMA operands.
  const int k_off = prow(l32) * S + hf * 8;   // + kb*32*S + ks*16
  const TrOffsets v_off = tr_lane_offsets<S>(lane);  // + (kb*32 + s*16)*S + db*32

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  // Row sums on the matrix core: a 32-row block of ones as one more A operand of
  // O^T += V^T P^T gives, in every register of lane l, sum_j P_lj over the same bf16
  // probabilities the numerator uses (the VALU row sum with v_dot2c_f32_bf16 ran
  // several times slower beside the other wave's MFMAs).
  f32x16 acc_l = f32x16{};
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  float m = -INFINITY;
  float mc = 0.f;                           // m * c, or 0 while m is unset
  const float c = p.scale_log2;
  const int lim = P + t;                    // this row may attend keys 0..lim

  // MFMA block of a phase: S^T = K Q^T of tile i (16 MFMAs at D = 128, one LDS read
  // each) and O^T += V^T P^T of tile i - 1 (16 MFMAs, two transposing reads each),
  // every read issued kFwdReadAhead MFMAs ahead of its MFMA.
  constexpr int NS = 2 * NKS, NPV = 4 * NDB;
  auto mblock = [&](auto do_s, auto do_pv, const uint16_t* kt, f32x16 (&st)[2],
                    const uint16_t* vt, const u32x4 (&pb)[4]) __attribute__((always_inline)) {
    constexpr bool kS = decltype(do_s)::value, kPV = decltype(do_pv)::value;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (kS) {
      st[0] = f32x16{};
      st[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int ks = i >> 1, kb = i & 1;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kt[k_off + kb * 32 * S + ks * 16]);
        st[kb] = mfma32(a, qreg[ks], st[kb]);
      }
    }
    if constexpr (kPV) {
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const bf16x8 a = lds_tr_operand<S>(vt, v_off, (i / NDB) * 16, (i % NDB) * 32);
        acc[i % NDB] = mfma32(a, __builtin_bit_cast(bf16x8, pb[i / NDB]), acc[i % NDB]);
      }
    }
    sched_chain2<kS ? NS : 0, 1, kPV ? NPV : 0, 2, kFwdReadAhead>();
    if constexpr (kPV) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) acc_l = mfma32(ones, __builtin_bit_cast(bf16x8, pb[s4]), acc_l);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (kS) {
      pin(st[0]);
      pin(st[1]);
    }
  };
  // Online softmax of one tile. The probabilities are taken against the running
  // reference m first; the exact row max is needed only when that reference is
  // unset or too low, which the tile's partial row sum shows: it exceeds
  // kSumLimit whenever some probability does. Then m is raised to the row max,
  // the accumulator rescaled and the tile's probabilities recomputed. Returns the
  // probabilities as the bf16 B operands of P V.
  // The VALU block runs alone on its SIMD half the time, so its dependency chains are
  // not hidden by another wave: the work goes in independent stages (every fma, then
  // every exp2, then the bf16 packs), each kept apart by a scheduling barrier.
  // Returns true if some probability of this lane exceeds kProbLimit (bf16 bits of
  // non-negative values order like unsigned integers).
  auto probs = [&](const f32x16 (&st)[2], u32x4 (&pb)[4]) __attribute__((always_inline)) {
    float x[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[kb * 16 + i] = fmaf(st[kb][i], c, -mc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]);
    __builtin_amdgcn_sched_barrier(0);
    // Word j of the packed probabilities holds scores 2j, 2j + 1 of the lane (x index
    // kb * 16 + i): word j % 4 of B operand j / 4.
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      uint32_t word;   // one v_cvt_pk_bf16_f32 (RNE) per pair, written in place
      asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(word) : "v"(x[2 * j]), "v"(x[2 * j + 1]));
      pb[j >> 2][j & 3] = word;
    }
    __builtin_amdgcn_sched_barrier(0);
    // (Each word is copied to a scalar before the bit_cast: hipcc reads element 0
    // when __builtin_bit_cast is applied to a subscripted vector element.)
    u16x2 mx[4];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t word = pb[j >> 2][j & 3];
      const u16x2 h = __builtin_bit_cast(u16x2, word);
      mx[j & 3] = j < 4 ? h : __builtin_elementwise_max(mx[j & 3], h);
    }
    mx[0] = __builtin_elementwise_max(__builtin_elementwise_max(mx[0], mx[1]),
                                      __builtin_elementwise_max(mx[2], mx[3]));
    return (mx[0][0] > kProbLimitBits) || (mx[0][1] > kProbLimitBits);
  };
  auto softmax = [&](f32x16 (&st)[2], int tile, u32x4 (&pb)[4]) __attribute__((always_inline)) {
    pin(st[0]);
    pin(st[1]);
    const int kbase = tile * BN;
    if (kbase + BN - 1 > P + t_min) {
      const int rel = lim - kbase - hf * 4;  // key kbase + o + hf*4 allowed iff o <= rel
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + (i >> 2) * 8 + (i & 3) > rel) st[kb][i] = -INFINITY;
    }
    const bool big = probs(st, pb);
    if (__builtin_amdgcn_ballot_w64(big || m == -INFINITY) != 0) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, st[kb][i]);
      const float mn = fmaxf(m, pair_max(mt));
      // alpha = 1 for rows that keep their max; 0 for rows leaving -inf.
      const float alpha = (mn == m) ? 1.f : __builtin_amdgcn_exp2f((m - mn) * c);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_l[i] *= alpha;
      m = mn;
      mc = (m == -INFINITY) ? 0.f : m * c;
      probs(st, pb);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) pin(pb[j]);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  const int n = te - tb;   // tiles of this workgroup (uniform)
  // Local tile l's rows are loaded into register slot l % 2 two phase pairs before
  // they are written to LDS (in the VALU phase of tile l - 1).
  if (n > 0) {
    stg.template issue<0>(tb);
    if (n > 1) stg.template issue<1>(tb + 1);
    stg.template store<0>(own0);
    if (n > 2) stg.template issue<0>(tb + 2);
  }
  phase_barrier();
  // One wait for every load so far (Q, and the next tiles' rows): without it the
  // compiler cannot tell at the loop header that Q has arrived, and its waits for Q
  // inside the MFMA block would also wait for the rows just requested.
  wait_global_loads();
  if (grp_w == 1) phase_barrier();   // group 1 runs one phase behind
  f32x16 st[2];
  u32x4 pb[4];
  // phase pair of tile 0: scores, then softmax (and staging of tile 1)
  if (n > 0) mblock(T_{}, F_{}, sm.k[0], st, sm.v[0], pb);
  phase_barrier();
  if (n > 0) {
    softmax(st, tb, pb);
    if (n > 1) stg.template store<1>(own1);
    if (n > 3) stg.template issue<1>(tb + 3);
  }
  phase_barrier();
  // Tiles 1 .. n - 1, two per trip so that the register slots are fixed.
  auto tile_pair = [&](auto slot, int i) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;   // slot of tile i + 1 = (i + 1) % 2
    const int cur = i & 1;
    mblock(T_{}, T_{}, sm.k[cur], st, sm.v[cur ^ 1], pb);
    phase_barrier();
    softmax(st, tb + i, pb);
    if (i + 1 < n) stg.template store<SL>(cur ? own0 : own1);
    if (i + 3 < n) stg.template issue<SL>(tb + i + 3);
    phase_barrier();
  };
  int i = 1;
  for (; i + 1 < n; i += 2) {
    tile_pair(std::integral_constant<int, 0>{}, i);       // i odd: tile i + 1 in slot 0
    tile_pair(std::integral_constant<int, 1>{}, i + 1);
  }
  if (i < n) tile_pair(std::integral_constant<int, 0>{}, i);
  // last phase: P V of the last tile
  if (n > 0) mblock(F_{}, T_{}, sm.k[0], st, sm.v[(n - 1) & 1], pb);
  phase_barrier();
  if (grp_w == 0) phase_barrier();   // matches group 1's extra barrier

  // Fused re-decode: the workgroups of this (window, KV head) share the append of
  // its chunk rows to cache rows [P_b, P_b + C). Those rows are never read by this
  // launch (the chunk's keys come from kc / vc), so the writes race with nothing.
  if (p.append) {
    const int nu = n_rb * SPL, u = split * n_rb + rb;
    const int64_t total = append_items<CT, D>(C);
    const int64_t crow0 = bh * p.cache.cap + P;
    for (int64_t it = (int64_t)u * NTHR + tid; it < total; it += (int64_t)nu * NTHR)
      append_item<CT, D>(it, C, p.kc + bh * C * D, p.vc + bh * C * D, p.wk, p.wv, p.wks,
                         p.wvs, crow0);
  }

  const float l_tot = acc_l[0];   // the row sum (both lanes of the row hold it)
  if (!row_ok) return;
  if (SPL == 1) {
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

// The same forward with each wave running its MFMA and softmax work back to back (no
// ping-pong): taken for F16 and q8_0 caches, whose conversion on staging makes the
// VALU phase the longer one, so the ping-pong's MFMA phase would wait on it.
template <int D, int CT>
__global__ __launch_bounds__(NTHR) void fwd_serial_kernel(FwdParams p) {
  __shared__ __align__(16) FwdLds<D> sm;
  constexpr int S = FwdLds<D>::S;
  constexpr int NKS = D / 16;   // k-steps over head_dim
  constexpr int NDB = D / 32;   // 32-row blocks of O^T

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  const int n_rb = p.plan.n_rb, SPL = p.plan.n_split;
  const int L = xcd_logical_id(blockIdx.x, p.plan.nblk);
  const int rb = L % n_rb;
  const int split = (L / n_rb) % SPL;
  const int grp = L / (n_rb * SPL);
  const int b = grp / p.Hkv, kv = grp % p.Hkv;
  const int G = p.G;
  const int C = (int)p.C;
  const int P = (int)window_prefix(p.plens, b, p.P);  // this window's prefix
  const int rows = G * C;
  constexpr int ROWS = 32 * NW;

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

  bf16x8 qreg[NKS];
  {
    const uint16_t* qp = p.q + qrow * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qreg[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }

  const int64_t bh = (int64_t)b * p.Hkv + kv;
  KVStager<CT, D, NTHR> stg(tid, p.cache, p.kc, p.vc, bh, P, p.C);

  // Per-lane LDS offsets of the MFMA operands.
  const int k_off = prow(l32) * S + hf * 8;   // + kb*32*S + ks*16
  const TrOffsets v_off = tr_lane_offsets<S>(lane);  // + (kb*32 + s*16)*S + db*32

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;
  float mc = 0.f;                           // m * c, or 0 while m is unset
  const float c = p.scale_log2;
  const int lim = P + t;                    // this row may attend keys 0..lim

  // MFMA blocks run at raised wave priority: when both waves of a SIMD are ready,
  // the one feeding the matrix core issues first and the other one's softmax VALU
  // work fills in behind it (measured: a few percent faster than equal priority).
  auto scores = [&](const uint16_t* kt, f32x16 (&st)[2]) {
    __builtin_amdgcn_s_setprio(1);
    bf16x8 a[NKS][2];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        a[ks][kb] = *reinterpret_cast<const bf16x8*>(&kt[k_off + kb * 32 * S + ks * 16]);
    st[0] = f32x16{};
    st[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) st[kb] = mfma32(a[ks][kb], qreg[ks], st[kb]);
    sched_ahead<2 * NKS, kFwdReadAhead, 1>();
    __builtin_amdgcn_s_setprio(0);
  };
  // Online softmax of one tile. The probabilities are taken against the running
  // reference m first; the exact row max is needed only when that reference is
  // unset or too low, which the tile's partial row sum shows: it exceeds
  // kSumLimit whenever some probability does. Then m is raised to the row max,
  // the accumulator rescaled and the tile's probabilities recomputed. Returns the
  // probabilities as the bf16 B operands of P V.
  auto probs = [&](const f32x16 (&st)[2], bf16x8 (&pb)[4]) {
    float lt = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const uint32_t w = pack_bf16(__builtin_amdgcn_exp2f(fmaf(st[kb][i], c, -mc)),
                                     __builtin_amdgcn_exp2f(fmaf(st[kb][i + 1], c, -mc)));
        lt = add_bf16_pair(w, lt);
        const bf16x2 pr = __builtin_bit_cast(bf16x2, w);
        pb[kb * 2 + (i >> 3)][i & 7] = pr[0];
        pb[kb * 2 + (i >> 3)][(i & 7) + 1] = pr[1];
      }
    return lt;
  };
  auto softmax = [&](f32x16 (&st)[2], int tile, bf16x8 (&pb)[4]) {
    const int kbase = tile * BN;
    if (kbase + BN - 1 > P + t_min) {
      const int rel = lim - kbase - hf * 4;  // key kbase + o + hf*4 allowed iff o <= rel
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + (i >> 2) * 8 + (i & 3) > rel) st[kb][i] = -INFINITY;
    }
    float lt = probs(st, pb);
    if (__builtin_amdgcn_ballot_w64(lt > kSumLimit || m == -INFINITY) != 0) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, st[kb][i]);
      const float mn = fmaxf(m, pair_max(mt));
      // alpha = 1 for rows that keep their max; 0 for rows leaving -inf.
      const float alpha = (mn == m) ? 1.f : __builtin_amdgcn_exp2f((m - mn) * c);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      m = mn;
      mc = (m == -INFINITY) ? 0.f : m * c;
      lt = probs(st, pb);
    }
    l += lt;
  };
  // P V operands: the first kPre are read before the softmax (they do not depend on
  // it), the rest kFwdReadAhead MFMAs ahead of their use.
  constexpr int NPV = 4 * NDB;
  constexpr int kPre = kFwdPvEarlyReads;
  auto pv_operand = [&](const uint16_t* vt, int i) __attribute__((always_inline)) {
    return lds_tr_operand<S>(vt, v_off, (i / NDB) * 16, (i % NDB) * 32);
  };
  auto pv_mfma = [&](const uint16_t* vt, const bf16x8 (&pb)[4], bf16x8 (&a)[NPV]) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = kPre; i < NPV; ++i) a[i] = pv_operand(vt, i);
#pragma unroll
    for (int i = 0; i < NPV; ++i) acc[i % NDB] = mfma32(a[i], pb[i / NDB], acc[i % NDB]);
    sched_ahead_after<NPV, kPre, kFwdReadAhead, 2>();
    __builtin_amdgcn_s_setprio(0);
  };

  if (tb < te) {
    stg.issue(tb);
    stg.store(sm.k[0], sm.v[0]);
    if (tb + 1 < te) stg.issue(tb + 1);
    __syncthreads();
  }
  wait_global_loads();
  for (int tile = tb; tile < te; ++tile) {
    const int cur = (tile - tb) & 1;
    f32x16 st[2];
    scores(sm.k[cur], st);
    bf16x8 pva[NPV];
#pragma unroll
    for (int i = 0; i < kPre; ++i) pva[i] = pv_operand(sm.v[cur], i);
    bf16x8 pb[4];
    softmax(st, tile, pb);
    pv_mfma(sm.v[cur], pb, pva);
    if (tile + 1 < te) {
      stg.store(sm.k[cur ^ 1], sm.v[cur ^ 1]);
      if (tile + 2 < te) stg.issue(tile + 2);
      __syncthreads();
    }
  }

  // Fused re-decode: the workgroups of this (window, KV head) share the append of
  // its chunk rows to cache rows [P_b, P_b + C). Those rows are never read by this
  // launch (the chunk's keys come from kc / vc), so the writes race with nothing.
  if (p.append) {
    const int nu = n_rb * SPL, u = split * n_rb + rb;
    const int64_t total = append_items<CT, D>(C);
    const int64_t crow0 = bh * p.cache.cap + P;
    for (int64_t it = (int64_t)u * NTHR + tid; it < total; it += (int64_t)nu * NTHR)
      append_item<CT, D>(it, C, p.kc + bh * C * D, p.vc + bh * C * D, p.wk, p.wv, p.wks,
                         p.wvs, crow0);
  }

  const float l_tot = pair_sum(l);
  if (!row_ok) return;
  if (SPL == 1) {
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
  if constexpr (CT == kBF16)
    hipLaunchKernelGGL((fwd_kernel<D, CT>), dim3(p.plan.nblk), dim3(NTHR), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_serial_kernel<D, CT>), dim3(p.plan.nblk), dim3(NTHR), 0, s, p);
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
