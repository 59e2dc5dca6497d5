// Internal interface between the C-ABI host layer (pka_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pka.h"

namespace pka {

// Tile geometry shared by host planning and kernels.
constexpr int kWavesPerBlock = 8;   // waves per forward / dQ workgroup (2 per SIMD)
constexpr int kBlocksPerCU = 1;     // resident forward / dQ workgroups per CU
constexpr int kRowsPerBlock = 32 * kWavesPerBlock;  // packed query rows per workgroup
constexpr int kKeysPerTile = 64;    // keys staged in LDS per step
constexpr int kDkvKeysPerBlock = 128;  // keys per dK/dV workgroup (4 waves x 32)
constexpr int kNumCUs = 256;        // MI355X compute units (8 XCDs x 32)
constexpr int kNumXCDs = 8;

// Pointers of one prefix cache; the element type is a template argument.
struct CacheRef {
  const void* k;
  const void* v;
  const uint16_t* ks;  // q8_0 scales (fp16 bits) or null
  const uint16_t* vs;
  int64_t cap;
};

// Work plan of the forward / dQ grids: units of (window, KV head, row block, split).
constexpr int kMaxDkvTable = 64;   // chunk key blocks with their own split counts

struct Plan {
  int n_rb;     // row blocks of kRowsPerBlock packed rows per (window, KV head)
  int n_split;  // prefix splits per row block
  int nblk;     // workgroups = B * Hkv * n_rb * n_split
  int n_dkv_split;  // backward only: query-row splits per dK/dV key block (the most
                    // of any block; > 1 means every block writes fp32 partials)
  // Chunk dK/dV with causal work per key block: block k is seen by G*(C - k*128)
  // packed rows, so it gets its own number of row splits. dkv_nkb > 0: block k
  // has splits [dkv_first[k], dkv_first[k + 1]) of the dkv_first[dkv_nkb] workgroups
  // of each (window, KV head). dkv_nkb == 0: every block has n_dkv_split splits.
  int dkv_nkb;
  int16_t dkv_first[kMaxDkvTable + 1];
  // backward only: 1 = the dK/dV units (one per key block, no row split) run in the
  // same grid as the dQ row blocks, on the CUs those leave idle; delta comes from a
  // launch before them
  int dkv_beside;
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  CacheRef cache;
  uint16_t* o;
  float* lse;
  float* ws_o;    // [n_split][B*Hq*C][D]  (only when n_split > 1)
  float* ws_lse;  // [n_split][B*Hq*C]
  int append;     // nonzero: also write the chunk's K/V to cache rows [P_b, P_b + C)
  void* wk;       // the cache as written by the append (same storage as `cache`)
  void* wv;
  uint16_t* wks;
  uint16_t* wvs;
  int B, Hq, Hkv, G;
  int64_t P, C;      // P: the (largest) prefix length
  const int32_t* plens;  // per-window prefix lengths (device) or null
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  Plan plan;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  CacheRef cache;
  const uint16_t* o;
  const float* lse;
  const uint16_t* d_o;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;   // [B*Hq*C]: caller's buffer or workspace
  float* ws_dq;   // [n_split][B*Hq*C][D] (only when n_split > 1)
  float* ws_dkv;  // [n_dkv_split][2][B*Hkv*NK][D] (only when n_dkv_split > 1)
  int64_t horizon;  // prefix gradient: the last `horizon` cache rows of each window
  float* dkp;       // prefix gradient outputs f32 [B][Hkv][horizon][D]
  float* dvp;
  int B, Hq, Hkv, G;
  int64_t P, C;
  const int32_t* plens;
  float scale;
  float scale_log2;
  Plan plan;
};

struct AppendParams {
  const uint16_t* k;  // bf16 [B][Hkv][C][D]
  const uint16_t* v;
  void* ck;
  void* cv;
  uint16_t* cks;
  uint16_t* cvs;
  int64_t rows;  // B * Hkv * C
  int64_t C, P, cap;
  const int32_t* plens;  // per-window prefix lengths (device) or null
  int Hkv;
  int D;
};

struct DequantParams {
  const int8_t* ck;
  const int8_t* cv;
  const uint16_t* cks;
  const uint16_t* cvs;
  float* out_f32;
  uint16_t* out_bf16;
  int64_t BH;   // batch * n_heads_kv
  int64_t row0, rows, cap;
  int D;
};

Plan plan_fwd(const pka_dims& d);
Plan plan_bwd(const pka_dims& d);
Plan plan_prefix_kv(const pka_dims& d, int64_t horizon);

// Profiling brackets (no-ops unless enabled).
void prof_begin(int kernel, hipStream_t s);
void prof_end(int kernel, hipStream_t s);

hipError_t launch_fwd(const FwdParams& p, int D, int cache_type, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, int D, int cache_type, hipStream_t s);
hipError_t launch_prefix_kv(const BwdParams& p, int D, int cache_type, hipStream_t s);
hipError_t launch_append(const AppendParams& p, int cache_type, hipStream_t s);
hipError_t launch_dequant(const DequantParams& p, hipStream_t s);

}  // namespace pka
