// Device helpers for gfx950 (CDNA4): MFMA wrappers, bf16/f16/q8_0 conversion,
// LDS layouts and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pka_internal.hpp"

namespace pka {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16). Lane l supplies A row l%32 and
// B column l%32, each with the 8 k-values (l/32)*8 .. +7 of the 16-wide k-step.
// The result holds column l%32 and rows (r/4)*8 + (l/32)*4 + r%4, r = 0..15.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b,
                                         const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Within a 32-row block of an MFMA result, lane half hf holds rows
// (r/4)*8 + hf*4 + r%4. Feeding registers 8s..8s+7 (k-step s) back as an operand
// whose lane half hf supplies k-values hf*8 + e makes k-position s*16 + hf*8 + e
// stand for row swap23(that position): bits 2 and 3 of the index exchanged. The
// other operand is staged in LDS with the same permutation (an involution).
__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Two floats -> packed bf16 pair (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Eight consecutive values of one key row, as loaded from HBM before conversion.
// Cache rows of F16/BF16 and chunk rows: 16 bytes. Q8_0 cache rows: 8 code bytes in
// .x/.y and the block's fp16 scale in .z.
struct RawRow8 {
  u32x4 w;
};

enum : int { kF16 = PKA_CACHE_F16, kBF16 = PKA_CACHE_BF16, kQ8 = PKA_CACHE_Q8_0 };

// Load 8 values (d0 .. d0+7) of key row j of the virtual key sequence
// [cache rows 0..P-1 ; chunk rows 0..C-1] of one (window, KV head).
// Returns true if the row is a cache row (needs conversion), false for a chunk row
// or a zero row beyond the sequence.
template <int CT, int D>
__device__ __forceinline__ bool load_row8(RawRow8& r, const void* cache_base,
                                          const uint16_t* cache_scale,
                                          const uint16_t* chunk_base, int64_t P,
                                          int64_t C, int64_t j, int d0) {
  if (j < P) {
    if constexpr (CT == kQ8) {
      const int8_t* src = static_cast<const int8_t*>(cache_base) + j * D + d0;
      u32x2 c = *reinterpret_cast<const u32x2*>(src);
      uint32_t s = cache_scale[j * (D / 32) + (d0 >> 5)];
      r.w = u32x4{c.x, c.y, s, 0u};
    } else {
      const uint16_t* src = static_cast<const uint16_t*>(cache_base) + j * D + d0;
      r.w = *reinterpret_cast<const u32x4*>(src);
    }
    return true;
  }
  if (j < P + C) {
    r.w = *reinterpret_cast<const u32x4*>(chunk_base + (j - P) * D + d0);
  } else {
    r.w = u32x4{0u, 0u, 0u, 0u};
  }
  return false;
}

// q8_0 dequantisation of 8 codes of one block: x = f32(d16) * q, the product of an
// 11-bit and an 8-bit significand, so exact in fp32 (an infinite scale gives +-inf,
// and NaN for a zero code, as the plain product does). The attention kernels and the
// dequantisation hook both call this one function. r.w.x / r.w.y hold the 8 code
// bytes (value e in byte e % 4 of word e / 4), r.w.z the block's fp16 scale bits.
__device__ __forceinline__ void dequant8_q8_0(const RawRow8& r, float (&x)[8]) {
  const float d = f16_to_f32(r.w.z & 0xffffu);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = e < 4 ? r.w.x : r.w.y;
    x[e] = d * (float)(int8_t)((w >> (8 * (e & 3))) & 0xffu);
  }
}

// Raw row -> 8 bf16 values packed in 4 dwords (element 2i in the low half of .i).
// F16 and q8_0 values are converted to fp32 exactly, then rounded to bf16 (RNE).
template <int CT>
__device__ __forceinline__ u32x4 to_bf16x8(const RawRow8& r, bool is_cache) {
  if (!is_cache || CT == kBF16) return r.w;
  if constexpr (CT == kF16) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = r.w[i];
      o[i] = pack_bf16(f16_to_f32(w & 0xffffu), f16_to_f32(w >> 16));
    }
    return o;
  } else {
    float x[8];
    dequant8_q8_0(r, x);
    return u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                 pack_bf16(x[6], x[7])};
  }
}

// Prefix length of window b: its entry of the optional per-window array, clamped to
// [0, P] (P: the largest prefix, which bounds every cache access), else P.
__device__ __forceinline__ int64_t window_prefix(const int32_t* plens, int b, int64_t P) {
  if (plens == nullptr) return P;
  const int64_t pb = plens[b];
  return pb < 0 ? 0 : (pb > P ? P : pb);
}

// Workgroup order: hardware dispatches workgroup i to XCD i % 8. Renumber so each
// XCD receives a contiguous range of logical ids; neighbouring logical ids read the
// same K/V tiles and so share that XCD's L2.
__device__ __forceinline__ int xcd_logical_id(int i, int nblk) {
  const int q = nblk / kNumXCDs;
  const int rem = nblk % kNumXCDs;
  const int x = i % kNumXCDs;
  const int k = i / kNumXCDs;
  return x * q + (x < rem ? x : rem) + k;
}

// Instruction order of an unrolled chain of N MFMAs whose A operands take R LDS
// reads each: the reads run PF MFMAs ahead of their use (scheduling-group barriers;
// masks 0x100 = LDS reads, 0x008 = MFMA). Without it the compiler issues each
// operand read right before its MFMA, and the wave waits out the LDS latency.
template <int I, int N, int R>
__device__ __forceinline__ void sched_rep_mr() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
    sched_rep_mr<I + 1, N, R>();
  }
}
template <int N, int PF, int R>
__device__ __forceinline__ void sched_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, R * PF, 0);
  sched_rep_mr<0, N - PF, R>();
  __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
}

// As sched_ahead, for a chain whose first PRE operands were read earlier (before
// other work): the remaining reads run PF MFMAs ahead.
template <int N, int PRE, int PF, int R>
__device__ __forceinline__ void sched_ahead_after() {
  constexpr int LEAD = PF > PRE ? PF - PRE : 0;   // reads to issue before the first MFMA
  if constexpr (LEAD > 0) __builtin_amdgcn_sched_group_barrier(0x100, R * LEAD, 0);
  sched_rep_mr<0, N - PRE - LEAD, R>();
  __builtin_amdgcn_sched_group_barrier(0x008, PRE + LEAD, 0);
}
// Read-ahead depths (MFMAs), measured: the forward's S and P V chains 6 (the first
// 4 P V operands read before the softmax); the dQ kernel's S / dP chains 4 and its
// dQ chain 3 (it has no registers for more).
constexpr int kFwdReadAhead = 6;
constexpr int kFwdPvEarlyReads = 4;
constexpr int kDqReadAheadSP = 4;
constexpr int kDqReadAheadDQ = 3;

// Wait until every global load this wave issued has returned (s_waitcnt vmcnt(0)).
// Used once after a kernel's prologue: the compiler cannot tell at the loop header
// whether the one-time operand loads (Q, dO) are still in flight, and otherwise
// inserts waits inside the loop that also stall on the next tile's prefetch.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Lane l and lane l ^ 32 hold the two halves of one row: sum / max of the pair,
// returned to both lanes (v_permlane32_swap, no LDS round trip).
__device__ __forceinline__ float pair_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum of a packed bf16 pair, accumulated in fp32 (v_dot2c_f32_bf16 with (1, 1)).
__device__ __forceinline__ float add_bf16_pair(uint32_t packed, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

// ---------------------------------------------------------------------------
// LDS tiles. Every tile is row-major (one token row of D bf16 per row) with a
// row stride of D + 8 elements, and the 16 rows of each aligned group are stored
// in the order prow(r): r = 4a + b (a, b < 4) lands in physical row 4b + a.
// Measured on gfx950 (SQ_LDS_BANK_CONFLICT of a probe of both access kinds), this
// layout makes both the 16-byte MFMA operand reads (lane -> one row, 8
// consecutive values) and the transposing reads below (16 lanes -> a 4-row x
// 16-column block) conflict-free; staging writes of whole rows by 16 consecutive
// lanes stay contiguous.
__device__ __forceinline__ int prow(int r) {
  return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef v4i16 __attribute__((address_space(3))) * lds_v4i16_ptr;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane p receives element p%4
// of the 8-byte pieces addressed by lanes p/4, p/4+4, p/4+8 and p/4+12. If lane q
// of the group addresses row R0 + q/4, columns C0 + 4(q%4) .. +3 of a row-major
// tile, lane p receives column C0 + p of rows R0 .. R0+3 (a 4x16 transpose).
__device__ __forceinline__ v4i16 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16_ptr)((__attribute__((address_space(3))) uint16_t*)(p)));
}

// The transposed MFMA operand of one 16-row k-step: lane (l32, hf) of the wave
// gets, for output row (column of the tile) C0 + l32, the 8 tile rows
// R0 + {0..3, 8..11} + 4 hf, in the order that matches registers 8s..8s+7 of an
// MFMA result (see swap23). R0 must be a multiple of 16 and C0 of 32.
struct TrOffsets {
  int lo, hi;  // per-lane element offsets of the two 4-row reads
};
template <int STRIDE>
__device__ __forceinline__ TrOffsets tr_lane_offsets(int lane) {
  const int q = lane & 15, hf = lane >> 5, h16 = (lane >> 4) & 1;
  const int col = h16 * 16 + (q & 3) * 4;
  const int y = hf * 4 + (q >> 2);
  return TrOffsets{prow(y) * STRIDE + col, prow(8 + y) * STRIDE + col};
}
template <int STRIDE>
__device__ __forceinline__ bf16x8 lds_tr_operand(const uint16_t* tile, const TrOffsets& o,
                                                 int r0, int c0) {
  const v4i16 lo = lds_read_tr(tile + o.lo + r0 * STRIDE + c0);
  const v4i16 hi = lds_read_tr(tile + o.hi + r0 * STRIDE + c0);
  const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// Staging of one tile of 64 keys of K and V, [cache rows 0..P-1 ; chunk rows],
// from HBM into two row-major LDS tiles (layout below). The work is 2 * NT tasks of
// 4 rows x 8 values (NT per tensor); thread tid takes tasks tid + s * NTHR. Loads
// go to registers first (issue) so that they overlap the compute of the current
// tile, and are converted to bf16 when written to LDS (store).
struct Task4 {
  u32x4 w[4];
  bool cache[4];
};

template <int CT, int D, int NTHR>
struct KVStager {
  static constexpr int BN = kKeysPerTile;
  static constexpr int CH = D / 8;
  static constexpr int NT = (BN / 4) * CH;             // tasks per tensor
  static constexpr int TPT = (2 * NT + NTHR - 1) / NTHR;  // task slots per thread
  static constexpr int ESZ = (CT == kQ8) ? 1 : 2;
  static constexpr int S = D + 8;

  const char* cbase[TPT];
  const uint16_t* cscale[TPT];
  const uint16_t* chunk[TPT];
  int tr0[TPT], td0[TPT];
  bool active[TPT], is_k[TPT];
  Task4 raw[TPT];
  int64_t P, C;
  int n_fast;  // tiles [0, n_fast) lie wholly in the cache

  __device__ __forceinline__ KVStager(int tid, const CacheRef& cache, const uint16_t* kc,
                                      const uint16_t* vc, int64_t bh, int64_t P_,
                                      int64_t C_) {
    P = P_;
    C = C_;
    n_fast = (int)(P_ / BN);
#pragma unroll
    for (int s = 0; s < TPT; ++s) {
      const int task = tid + s * NTHR;
      is_k[s] = task < NT;
      active[s] = task < 2 * NT;
      const int tk = is_k[s] ? task : task - NT;
      tr0[s] = (tk / CH) * 4;
      td0[s] = (tk % CH) * 8;
      cbase[s] = static_cast<const char*>(is_k[s] ? cache.k : cache.v) + bh * cache.cap * D * ESZ;
      cscale[s] = (CT == kQ8) ? (is_k[s] ? cache.ks : cache.vs) + bh * cache.cap * (D / 32)
                              : nullptr;
      chunk[s] = (is_k[s] ? kc : vc) + bh * C_ * D;
    }
  }

  // Load the K rows of tile tk and the V rows of tile tv into registers; a
  // negative index loads nothing for that tensor. fast: both tiles lie wholly in
  // the cache (uniform base pointer, no per-row checks).
  template <bool FAST>
  __device__ __forceinline__ void issue(int tk, int tv) {
#pragma unroll
    for (int s = 0; s < TPT; ++s) {
      if (!active[s]) continue;
      const int tile = is_k[s] ? tk : tv;
      if (!FAST && tile < 0) continue;
      Task4& t = raw[s];
      if (FAST || tile < n_fast) {
        const char* base = cbase[s] + (int64_t)tile * BN * D * ESZ;
        const char* sbase = reinterpret_cast<const char*>(cscale[s] + (int64_t)tile * BN * (D / 32));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = tr0[s] + i;
          if constexpr (CT == kQ8) {
            const u32x2 c = *reinterpret_cast<const u32x2*>(base + r * D + td0[s]);
            const uint32_t sc =
                *reinterpret_cast<const uint16_t*>(sbase + (r * (D / 32) + (td0[s] >> 5)) * 2);
            t.w[i] = u32x4{c.x, c.y, sc, 0u};
          } else {
            t.w[i] = *reinterpret_cast<const u32x4*>(base + (r * D + td0[s]) * 2);
          }
          t.cache[i] = true;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          RawRow8 r;
          t.cache[i] = load_row8<CT, D>(r, cbase[s], cscale[s], chunk[s], P, C,
                                        (int64_t)tile * BN + tr0[s] + i, td0[s]);
          t.w[i] = r.w;
        }
      }
    }
  }
  __device__ __forceinline__ void issue(int tile) { issue<false>(tile, tile); }

  // Convert and write the loaded rows; a null tile skips that tensor.
  __device__ __forceinline__ void store(uint16_t* ktile, uint16_t* vtile) const {
#pragma unroll
    for (int s = 0; s < TPT; ++s) {
      if (!active[s]) continue;
      uint16_t* tile = is_k[s] ? ktile : vtile;
      if (tile == nullptr) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        RawRow8 r;
        r.w = raw[s].w[i];
        *reinterpret_cast<u32x4*>(&tile[prow(tr0[s] + i) * S + td0[s]]) =
            to_bf16x8<CT>(r, raw[s].cache[i]);
      }
    }
  }
};


// ---------------------------------------------------------------------------
// Staging of ONE tensor (K or V) of the key sequence [cache rows 0..P-1 ; chunk rows]
// in tiles of 64 keys, by NTHR threads (one 4-wave group of a ping-pong workgroup).
// Thread g takes RPT consecutive rows of one 8-value column chunk. Loads go to one of
// NSLOT register slots (issue), and are converted and written to LDS later (store),
// so NSLOT tiles can be in flight; the slot is a template argument so that the
// registers stay registers.
template <int CT, int D, int NTHR, int NSLOT = 1>
struct TileStager {
  static constexpr int BN = kKeysPerTile;
  static constexpr int CH = D / 8;                 // 8-value chunks per row
  static constexpr int RPT = BN * CH / NTHR;       // rows per thread
  static constexpr int ESZ = (CT == kQ8) ? 1 : 2;
  static constexpr int S = D + 8;
  static_assert(RPT >= 1 && BN * CH == RPT * NTHR, "tile does not split evenly");

  const char* cbase;        // this (window, KV head)'s cache rows of the tensor
  const uint16_t* cscale;   // q8_0 scales or null
  const uint16_t* chunk;    // the chunk's own rows (bf16 [C][D])
  int tr0, td0;
  int64_t P, C;
  int n_fast;               // tiles [0, n_fast) lie wholly in the cache
  u32x4 raw[NSLOT][RPT];
  bool in_cache[NSLOT][RPT];

  __device__ __forceinline__ TileStager(int g, const void* cache_base, const uint16_t* scale_base,
                                        const uint16_t* chunk_base, int64_t bh, int64_t cap,
                                        int64_t P_, int64_t C_) {
    P = P_;
    C = C_;
    n_fast = (int)(P_ / BN);
    tr0 = (g / CH) * RPT;
    td0 = (g % CH) * 8;
    cbase = static_cast<const char*>(cache_base) + bh * cap * D * ESZ;
    cscale = (CT == kQ8) ? scale_base + bh * cap * (D / 32) : nullptr;
    chunk = chunk_base + bh * C_ * D;
  }

  // Load this thread's rows of tile `tile` into register slot SL.
  template <int SL = 0>
  __device__ __forceinline__ void issue(int tile) {
    if (tile < n_fast) {
      const char* base = cbase + (int64_t)tile * BN * D * ESZ;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = tr0 + i;
        if constexpr (CT == kQ8) {
          const u32x2 c = *reinterpret_cast<const u32x2*>(base + r * D + td0);
          const uint32_t sc = cscale[((int64_t)tile * BN + r) * (D / 32) + (td0 >> 5)];
          raw[SL][i] = u32x4{c.x, c.y, sc, 0u};
        } else {
          raw[SL][i] = *reinterpret_cast<const u32x4*>(base + (r * D + td0) * 2);
        }
        in_cache[SL][i] = true;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        RawRow8 r;
        in_cache[SL][i] = load_row8<CT, D>(r, cbase, cscale, chunk, P, C,
                                           (int64_t)tile * BN + tr0 + i, td0);
        raw[SL][i] = r.w;
      }
    }
  }

  // Convert the rows of slot SL to bf16 and write them to a row-major LDS tile.
  template <int SL = 0>
  __device__ __forceinline__ void store(uint16_t* tile) const {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      RawRow8 r;
      r.w = raw[SL][i];
      *reinterpret_cast<u32x4*>(&tile[prow(tr0 + i) * S + td0]) = to_bf16x8<CT>(r, in_cache[SL][i]);
    }
  }
};

// Instruction order of a block of N0 MFMAs whose A operands take R0 LDS reads each,
// followed by N1 MFMAs taking R1 reads each: every read is issued PF MFMAs before the
// MFMA that uses it (scheduling-group barriers: 0x008 MFMA, 0x100 LDS read).
template <int K, int N0, int R0, int N1, int R1, int PF>
__device__ __forceinline__ void sched_chain2_step() {
  if constexpr (K < N0 + N1) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int J = K + PF;
    if constexpr (J < N0 + N1) __builtin_amdgcn_sched_group_barrier(0x100, J < N0 ? R0 : R1, 0);
    sched_chain2_step<K + 1, N0, R0, N1, R1, PF>();
  }
}
template <int J, int N0, int R0, int N1, int R1, int PF>
__device__ __forceinline__ void sched_chain2_lead() {
  if constexpr (J < PF && J < N0 + N1) {
    __builtin_amdgcn_sched_group_barrier(0x100, J < N0 ? R0 : R1, 0);
    sched_chain2_lead<J + 1, N0, R0, N1, R1, PF>();
  }
}
template <int N0, int R0, int N1, int R1, int PF>
__device__ __forceinline__ void sched_chain2() {
  sched_chain2_lead<0, N0, R0, N1, R1, PF>();
  sched_chain2_step<0, N0, R0, N1, R1, PF>();
}

// Phase boundary of a ping-pong workgroup: LDS writes of this phase complete, then
// every wave of the workgroup meets. Nothing is scheduled across it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

// Pin a value at this point of the instruction stream: it must be computed before it
// and may not be read by anything placed before it (an empty asm that "modifies" it).
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// ---------------------------------------------------------------------------
// Cache writes of the chunk's K/V rows (re-decode into the cache).
// q8_0 block (32 consecutive values of one token row along head_dim):
//   amax = max|x|; d = amax / 127 (IEEE fp32 division; the library is built without
//   fast-math, so '/' is correctly rounded); scale = fp16(d) (RNE);
//   code = clamp(round_half_away_from_zero(x / d), -127, 127) using the fp32 d;
//   amax == 0 stores scale 0 and codes 0. Dequantised value = f32(scale) * code.
__device__ __forceinline__ void q8_0_block(const uint16_t* src, int8_t* dst_codes,
                                           uint16_t* dst_scale) {
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
  reinterpret_cast<u32x4*>(dst_codes)[0] = q[0];
  reinterpret_cast<u32x4*>(dst_codes)[1] = q[1];
  *dst_scale = f32_to_f16_bits(d);
}

// 8 bf16 values -> the 16-bit cache type: F16 (round to nearest even) or a copy.
template <int CT>
__device__ __forceinline__ u32x4 to_cache16(const u32x4& w) {
  if constexpr (CT == kF16) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)f32_to_f16_bits(bf16_to_f32(w[e] & 0xffffu)) |
             ((uint32_t)f32_to_f16_bits(bf16_to_f32(w[e] >> 16)) << 16);
    return o;
  } else {
    return w;
  }
}

// Number of work items of the append of one (window, KV head): q8_0 blocks of 32
// values or 16-bit chunks of 8 values, K rows first, then V rows.
template <int CT, int D>
__host__ __device__ constexpr int64_t append_items(int64_t C) {
  return 2 * C * (CT == kQ8 ? D / 32 : D / 8);
}

// Item `it` of the append of one (window, KV head) whose chunk rows start at kc / vc
// (bf16 [C][D]) and whose first written cache row is `crow0` (element offset of row
// P_b of this window and KV head, in rows).
template <int CT, int D>
__device__ __forceinline__ void append_item(int64_t it, int64_t C, const uint16_t* kc,
                                            const uint16_t* vc, void* ck, void* cv,
                                            uint16_t* cks, uint16_t* cvs, int64_t crow0) {
  constexpr int PER = CT == kQ8 ? D / 32 : D / 8;
  const int64_t half = C * PER;
  const bool is_v = it >= half;
  const int64_t i = is_v ? it - half : it;
  const int64_t tok = i / PER;
  const int part = (int)(i - tok * PER);
  const int64_t crow = crow0 + tok;
  if constexpr (CT == kQ8) {
    const uint16_t* src = (is_v ? vc : kc) + tok * D + part * 32;
    int8_t* dst = static_cast<int8_t*>(is_v ? cv : ck) + crow * D + part * 32;
    q8_0_block(src, dst, (is_v ? cvs : cks) + crow * (D / 32) + part);
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>((is_v ? vc : kc) + tok * D + part * 8);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(is_v ? cv : ck) + crow * D + part * 8) =
        to_cache16<CT>(w);
  }
}

}  // namespace pka
