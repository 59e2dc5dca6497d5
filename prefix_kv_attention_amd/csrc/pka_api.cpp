// C-ABI host layer of libpka: argument validation (before any HIP call), work
// planning, workspace layout and kernel launches. See include/pka.h for the
// contract of every entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "pka_internal.hpp"
#include "row_sparse.hpp"

namespace pka {
namespace {

thread_local char g_last_error[512] = "";

pka_status fail(pka_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

pka_status hip_fail(hipError_t e, const char* what) {
  return fail(PKA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

constexpr int64_t kMaxChunk = 65536;
constexpr int64_t kMaxSeq = 2147483647LL;
// Q / dO rows of one KV head in the backward, with room for one step of padding rows.
constexpr int64_t kMaxGroupRowBytes = (1LL << 32) - (1LL << 20);

pka_status check_dims(const pka_dims* d) {
  if (!d) return fail(PKA_ERR_NULL, "dims is NULL");
  if (d->batch < 1 || d->n_heads_q < 1 || d->n_heads_kv < 1)
    return fail(PKA_ERR_DIMS, "batch, n_heads_q and n_heads_kv must be >= 1");
  if (d->n_heads_q % d->n_heads_kv != 0)
    return fail(PKA_ERR_DIMS, "n_heads_q (%d) is not a multiple of n_heads_kv (%d)",
                d->n_heads_q, d->n_heads_kv);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PKA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->prefix_len < 0) return fail(PKA_ERR_DIMS, "prefix_len < 0");
  if (d->chunk_len < 1 || d->chunk_len > kMaxChunk)
    return fail(PKA_ERR_DIMS, "chunk_len must be in [1, %lld]", (long long)kMaxChunk);
  if (d->prefix_len > kMaxSeq - d->chunk_len)
    return fail(PKA_ERR_DIMS, "prefix_len + chunk_len exceeds 2^31 - 1");
  const int64_t nrow = (int64_t)d->batch * d->n_heads_q * d->chunk_len;
  if (nrow > kMaxSeq) return fail(PKA_ERR_DIMS, "batch * n_heads_q * chunk_len exceeds 2^31 - 1");
  if ((int64_t)(d->n_heads_q / d->n_heads_kv) * d->chunk_len > kMaxSeq)
    return fail(PKA_ERR_DIMS, "group * chunk_len exceeds 2^31 - 1");
  if (!(d->softmax_scale > 0.f) || !std::isfinite(d->softmax_scale))
    return fail(PKA_ERR_DIMS, "softmax_scale must be finite and > 0");
  if ((reinterpret_cast<uintptr_t>(d->prefix_lens) & 3u) != 0)
    return fail(PKA_ERR_ALIGN, "prefix_lens not 4-byte aligned");
  return PKA_OK;
}

// The backward kernels address the Q / dO rows of one KV head's query heads (G * C rows
// of D bf16 values) with 32-bit byte offsets.
pka_status check_group_rows(const pka_dims* d) {
  const int64_t bytes =
      (int64_t)(d->n_heads_q / d->n_heads_kv) * d->chunk_len * d->head_dim * 2;
  if (bytes > kMaxGroupRowBytes)
    return fail(PKA_ERR_DIMS,
                "the query rows of one KV head (group * chunk_len * head_dim * 2 bytes) "
                "must stay below 4 GiB");
  return PKA_OK;
}

// rows_needed: cache rows the call addresses (P for attention, P + C for appends).
pka_status check_cache(const pka_cache* c, const pka_dims* d, int64_t rows_needed,
                       bool writes) {
  if (!c) return fail(PKA_ERR_NULL, "cache is NULL");
  if (c->type != PKA_CACHE_F16 && c->type != PKA_CACHE_BF16 && c->type != PKA_CACHE_Q8_0)
    return fail(PKA_ERR_UNSUPPORTED, "unknown cache type %d", c->type);
  if (c->head_dim != d->head_dim)
    return fail(PKA_ERR_DIMS, "cache head_dim %d != dims head_dim %d", c->head_dim, d->head_dim);
  if (c->capacity < 0) return fail(PKA_ERR_DIMS, "cache capacity < 0");
  if (rows_needed > c->capacity)
    return fail(PKA_ERR_CAPACITY, "cache capacity %lld < %lld rows addressed",
                (long long)c->capacity, (long long)rows_needed);
  if (rows_needed > 0 || writes) {
    if (!c->k || !c->v) return fail(PKA_ERR_NULL, "cache k/v is NULL");
    if (!aligned16(c->k) || !aligned16(c->v))
      return fail(PKA_ERR_ALIGN, "cache k/v not 16-byte aligned");
    if (c->type == PKA_CACHE_Q8_0) {
      if (!c->k_scale || !c->v_scale) return fail(PKA_ERR_NULL, "q8_0 cache scales are NULL");
      if (!aligned16(c->k_scale) || !aligned16(c->v_scale))
        return fail(PKA_ERR_ALIGN, "q8_0 cache scales not 16-byte aligned");
    }
  }
  return PKA_OK;
}

pka_status check_ptrs(std::initializer_list<const void*> ptrs, const char* names) {
  for (const void* ptr : ptrs) {
    if (!ptr) return fail(PKA_ERR_NULL, "a required tensor pointer is NULL (%s)", names);
    if (!aligned16(ptr)) return fail(PKA_ERR_ALIGN, "a tensor pointer is not 16-byte aligned (%s)", names);
  }
  return PKA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

CacheRef cache_ref(const pka_cache* c) {
  CacheRef r;
  r.k = c->k;
  r.v = c->v;
  r.ks = static_cast<const uint16_t*>(c->k_scale);
  r.vs = static_cast<const uint16_t*>(c->v_scale);
  r.cap = c->capacity;
  return r;
}

// ---------------------------------------------------------------- profiling
constexpr int kMaxRecords = 65536;
struct ProfSlot {
  std::vector<hipEvent_t> begin, end;  // pooled events, reused across resets
  int64_t used = 0;
  int64_t dropped = 0;
  bool open = false;                   // a begin event was recorded, its end not yet
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::atomic<uint32_t> g_prof_mask{0xFFFFFFFFu};   // kernels bracketed while enabled
ProfSlot g_prof[PKA_KERNEL_COUNT];

}  // namespace

void prof_begin(int kernel, hipStream_t s) {
  if (!g_prof_on.load(std::memory_order_relaxed) ||
      !((g_prof_mask.load(std::memory_order_relaxed) >> kernel) & 1u))
    return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfSlot& sl = g_prof[kernel];
  if (sl.used >= kMaxRecords) {
    ++sl.dropped;
    return;
  }
  if ((int64_t)sl.begin.size() <= sl.used) {
    // Timing-only events: without the system-scope fence, recording one does not
    // write back and invalidate the caches between the kernels it separates (with the
    // fence, each record left a ~6 us gap before the next kernel).
    hipEvent_t a, b;
    if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return;
    if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
      (void)hipEventDestroy(a);
      return;
    }
    sl.begin.push_back(a);
    sl.end.push_back(b);
  }
  sl.open = hipEventRecord(sl.begin[sl.used], s) == hipSuccess;
}

void prof_end(int kernel, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfSlot& sl = g_prof[kernel];
  if (!sl.open) return;   // its begin was not recorded (off, not selected, or full)
  sl.open = false;
  if (hipEventRecord(sl.end[sl.used], s) == hipSuccess) ++sl.used;
}

// One row block is kRowsPerBlock packed rows of one (window, KV head) and runs as
// one 8-wave workgroup, one per CU. When these units are fewer than the CUs, the
// key tiles are split so that units x splits still fits in one round of 256
// workgroups; each split keeps at least 8 tiles so the merge stays small next to
// the work.
static Plan make_plan(const pka_dims& d) {
  Plan pl{};
  const int64_t G = d.n_heads_q / d.n_heads_kv;
  pl.n_rb = (int)((G * d.chunk_len + kRowsPerBlock - 1) / kRowsPerBlock);
  const int64_t units = (int64_t)d.batch * d.n_heads_kv * pl.n_rb;
  int64_t split = 1;
  if (units < kNumCUs * kBlocksPerCU) {
    split = kNumCUs * kBlocksPerCU / units;
    const int64_t min_tiles = (d.prefix_len + 1 + kKeysPerTile - 1) / kKeysPerTile;
    const int64_t max_split = min_tiles / 8 > 1 ? min_tiles / 8 : 1;
    if (split > max_split) split = max_split;
    if (split > 16) split = 16;
  }
  pl.n_split = (int)split;
  pl.nblk = (int)(units * split);
  pl.n_dkv_split = 1;
  return pl;
}

Plan plan_fwd(const pka_dims& d) { return make_plan(d); }

// dK/dV: one unit per (window, KV head, block of kDkvKeysPerBlock chunk keys). When
// units are fewer than the CUs, they are split over disjoint ranges of query rows
// (each split keeps >= 2 steps of 64 rows, at most 16 splits) and the fp32 partials
// are summed afterwards. Key block k is seen only by the rows of tokens >= its first
// key, so the splits go where the rows are: starting from one per block, each
// further split of the CU budget goes to the block whose workgroups have the most
// steps (the first such block on ties).
Plan plan_bwd(const pka_dims& d) {
  Plan pl = make_plan(d);
  const int64_t G = d.n_heads_q / d.n_heads_kv;
  const int64_t nkb = (d.chunk_len + kDkvKeysPerBlock - 1) / kDkvKeysPerBlock;
  const int64_t groups = (int64_t)d.batch * d.n_heads_kv;
  const int64_t units = groups * nkb;
  pl.n_dkv_split = 1;
  pl.dkv_nkb = 0;
  pl.dkv_beside = 0;
  // Beside the dQ row blocks: when every unit (one per key block, all its rows) finds
  // an idle CU at the start and its steps (64 rows each) are no more than one dQ
  // workgroup's key tiles (the two cost about the same), the units finish inside the
  // dQ launch. Units that wait for a CU are not started on the ones the first units
  // free (measured), so the rule requires one round.
  if (pl.nblk < kNumCUs) {
    const int64_t idle = kNumCUs - pl.nblk;
    const int64_t unit_steps = (G * d.chunk_len + 63) / 64;
    const int64_t n_tiles = (d.prefix_len + d.chunk_len + kKeysPerTile - 1) / kKeysPerTile;
    const int64_t dq_tiles = (n_tiles + pl.n_split - 1) / pl.n_split;
    if (units <= idle && unit_steps <= dq_tiles) {
      pl.dkv_beside = 1;
      return pl;
    }
  }
  if (units >= kNumCUs) return pl;
  if (nkb <= kMaxDkvTable) {
    int64_t steps[kMaxDkvTable], cnt[kMaxDkvTable];
    for (int64_t k = 0; k < nkb; ++k) {
      steps[k] = (G * (d.chunk_len - k * kDkvKeysPerBlock) + 63) / 64;
      cnt[k] = 1;
    }
    for (int64_t left = kNumCUs / groups - nkb; left > 0; --left) {
      int64_t best = -1, best_load = 0;
      for (int64_t k = 0; k < nkb; ++k) {
        const int64_t cap = steps[k] / 2 < 16 ? steps[k] / 2 : 16;
        if (cnt[k] >= cap) continue;
        const int64_t load = (steps[k] + cnt[k] - 1) / cnt[k];
        if (load > best_load) {
          best = k;
          best_load = load;
        }
      }
      if (best < 0) break;
      ++cnt[best];
    }
    int64_t first = 0, most = 1;
    for (int64_t k = 0; k < nkb; ++k) {
      pl.dkv_first[k] = (int16_t)first;
      first += cnt[k];
      if (cnt[k] > most) most = cnt[k];
    }
    pl.dkv_first[nkb] = (int16_t)first;
    pl.dkv_nkb = (int)nkb;
    pl.n_dkv_split = (int)most;
    return pl;
  }
  int64_t split = kNumCUs / units;
  const int64_t max_steps = (G * d.chunk_len + 63) / 64;
  const int64_t max_split = max_steps / 2 > 1 ? max_steps / 2 : 1;
  if (split > max_split) split = max_split;
  if (split > 16) split = 16;
  pl.n_dkv_split = (int)split;
  return pl;
}

// Prefix gradient: one unit per (window, KV head, block of 128 prefix keys of the
// horizon), split over query rows like the chunk dK/dV when units are few.
Plan plan_prefix_kv(const pka_dims& d, int64_t horizon) {
  Plan pl{};
  pl.n_rb = 0;
  pl.n_split = 1;
  pl.nblk = 0;
  const int64_t G = d.n_heads_q / d.n_heads_kv;
  const int64_t nkb = (horizon + kDkvKeysPerBlock - 1) / kDkvKeysPerBlock;
  const int64_t units = (int64_t)d.batch * d.n_heads_kv * nkb;
  int64_t split = 1;
  if (units > 0 && units < kNumCUs) {
    split = kNumCUs / units;
    const int64_t max_steps = (G * d.chunk_len + 63) / 64;
    const int64_t max_split = max_steps / 2 > 1 ? max_steps / 2 : 1;
    if (split > max_split) split = max_split;
    if (split > 16) split = 16;
  }
  pl.n_dkv_split = (int)split;
  return pl;
}

}  // namespace pka

using namespace pka;

extern "C" {

const char* pka_status_string(pka_status st) {
  switch (st) {
    case PKA_OK: return "ok";
    case PKA_ERR_NULL: return "a required pointer is NULL";
    case PKA_ERR_DIMS: return "inconsistent or out-of-range dimensions";
    case PKA_ERR_UNSUPPORTED: return "unsupported head_dim or cache type";
    case PKA_ERR_CAPACITY: return "cache capacity too small";
    case PKA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PKA_ERR_WORKSPACE: return "workspace missing or too small";
    case PKA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* pka_last_error(void) { return g_last_error; }

size_t pka_fwd_workspace_bytes(const pka_dims* dims) {
  if (check_dims(dims) != PKA_OK) return 0;
  const Plan pl = plan_fwd(*dims);
  if (pl.n_split == 1) return 0;
  const size_t nrow = (size_t)dims->batch * dims->n_heads_q * dims->chunk_len;
  return align256((size_t)pl.n_split * nrow * dims->head_dim * 4) +
         align256((size_t)pl.n_split * nrow * 4);
}

size_t pka_bwd_workspace_bytes(const pka_dims* dims) {
  if (check_dims(dims) != PKA_OK) return 0;
  const Plan pl = plan_bwd(*dims);
  const size_t nrow = (size_t)dims->batch * dims->n_heads_q * dims->chunk_len;
  size_t bytes = align256(nrow * 4);  // delta
  if (pl.n_split > 1) bytes += align256((size_t)pl.n_split * nrow * dims->head_dim * 4);
  if (pl.n_dkv_split > 1)
    bytes += align256((size_t)pl.n_dkv_split * 2 * dims->batch * dims->n_heads_kv *
                      dims->chunk_len * dims->head_dim * 4);
  return bytes;
}

static pka_status fwd_common(const pka_dims* dims, const void* q, const void* k,
                             const void* v, const pka_cache* cache, void* o, float* lse,
                             void* ws, size_t ws_bytes, pka_stream_t stream, bool append) {
  g_last_error[0] = 0;
  pka_status st;
  if ((st = check_dims(dims)) != PKA_OK) return st;
  if ((st = check_ptrs({q, k, v, o, lse}, "q, k, v, o, lse")) != PKA_OK) return st;
  const int64_t rows = dims->prefix_len + (append ? dims->chunk_len : 0);
  if ((st = check_cache(cache, dims, rows, append)) != PKA_OK) return st;
  const size_t need = pka_fwd_workspace_bytes(dims);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(PKA_ERR_WORKSPACE, "forward needs %zu workspace bytes, got %zu", need,
                  ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(PKA_ERR_ALIGN, "workspace not 16-byte aligned");
  }
  FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.kc = static_cast<const uint16_t*>(k);
  p.vc = static_cast<const uint16_t*>(v);
  p.cache = cache_ref(cache);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = dims->batch;
  p.Hq = dims->n_heads_q;
  p.Hkv = dims->n_heads_kv;
  p.G = dims->n_heads_q / dims->n_heads_kv;
  p.P = dims->prefix_len;
  p.plens = dims->prefix_lens;
  p.C = dims->chunk_len;
  p.scale = dims->softmax_scale;
  p.scale_log2 = (float)((double)dims->softmax_scale * 1.4426950408889634);
  p.plan = plan_fwd(*dims);
  if (p.plan.n_split > 1) {
    const size_t nrow = (size_t)p.B * p.Hq * p.C;
    p.ws_o = static_cast<float*>(ws);
    p.ws_lse = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        align256((size_t)p.plan.n_split * nrow * dims->head_dim * 4));
  }
  if (append) {
    p.append = 1;
    p.wk = cache->k;
    p.wv = cache->v;
    p.wks = static_cast<uint16_t*>(cache->k_scale);
    p.wvs = static_cast<uint16_t*>(cache->v_scale);
  }
  hipError_t e = launch_fwd(p, dims->head_dim, cache->type, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, append ? "chunk_attn_fwd_append launch"
                                                 : "chunk_attn_fwd launch");
  return PKA_OK;
}

pka_status pka_chunk_attn_fwd(const pka_dims* dims, const void* q, const void* k,
                              const void* v, const pka_cache* cache, void* o, float* lse,
                              void* ws, size_t ws_bytes, pka_stream_t stream) {
  return fwd_common(dims, q, k, v, cache, o, lse, ws, ws_bytes, stream, false);
}

pka_status pka_chunk_attn_fwd_append(const pka_dims* dims, const void* q, const void* k,
                                     const void* v, const pka_cache* cache, void* o,
                                     float* lse, void* ws, size_t ws_bytes,
                                     pka_stream_t stream) {
  return fwd_common(dims, q, k, v, cache, o, lse, ws, ws_bytes, stream, true);
}

pka_status pka_chunk_attn_bwd(const pka_dims* dims, const void* q, const void* k,
                              const void* v, const pka_cache* cache, const void* o,
                              const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                              float* delta, void* ws, size_t ws_bytes, pka_stream_t stream) {
  g_last_error[0] = 0;
  pka_status st;
  if ((st = check_dims(dims)) != PKA_OK) return st;
  if ((st = check_group_rows(dims)) != PKA_OK) return st;
  if ((st = check_ptrs({q, k, v, o, lse, d_o, dq, dk, dv}, "q, k, v, o, lse, d_o, dq, dk, dv")) !=
      PKA_OK)
    return st;
  if (delta && !aligned16(delta)) return fail(PKA_ERR_ALIGN, "delta not 16-byte aligned");
  if ((st = check_cache(cache, dims, dims->prefix_len, false)) != PKA_OK) return st;
  const size_t need = pka_bwd_workspace_bytes(dims);
  if (!ws || ws_bytes < need)
    return fail(PKA_ERR_WORKSPACE, "backward needs %zu workspace bytes, got %zu", need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(PKA_ERR_ALIGN, "workspace not 16-byte aligned");
  BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.kc = static_cast<const uint16_t*>(k);
  p.vc = static_cast<const uint16_t*>(v);
  p.cache = cache_ref(cache);
  p.o = static_cast<const uint16_t*>(o);
  p.lse = lse;
  p.d_o = static_cast<const uint16_t*>(d_o);
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.B = dims->batch;
  p.Hq = dims->n_heads_q;
  p.Hkv = dims->n_heads_kv;
  p.G = dims->n_heads_q / dims->n_heads_kv;
  p.P = dims->prefix_len;
  p.plens = dims->prefix_lens;
  p.C = dims->chunk_len;
  p.scale = dims->softmax_scale;
  p.scale_log2 = (float)((double)dims->softmax_scale * 1.4426950408889634);
  p.plan = plan_bwd(*dims);
  const size_t nrow = (size_t)p.B * p.Hq * p.C;
  float* ws_delta = static_cast<float*>(ws);
  p.delta = delta ? delta : ws_delta;
  size_t off = align256(nrow * 4);
  if (p.plan.n_split > 1) {
    p.ws_dq = reinterpret_cast<float*>(static_cast<char*>(ws) + off);
    off += align256((size_t)p.plan.n_split * nrow * dims->head_dim * 4);
  }
  if (p.plan.n_dkv_split > 1) p.ws_dkv = reinterpret_cast<float*>(static_cast<char*>(ws) + off);
  hipError_t e = launch_bwd(p, dims->head_dim, cache->type, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "chunk_attn_bwd launch");
  return PKA_OK;
}

// ---------------------------------------------------------------- allocation-free bwd
// The backward's workspace in device memory that the library owns: one file-scope
// array per GPU, which that GPU holds until the process ends. In host code `scratch`
// names a host-side stand-in, never the device memory, so its device address is looked
// up once per device (with that device current) and only that address is used.
namespace {
constexpr size_t kScratchBytes = PKA_BWD_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pka_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKA_ERR_UNSUPPORTED, "device %d beyond the %d the library supports", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKA_OK;
}
}  // namespace

pka_status pka_chunk_attn_bwd_noalloc(const pka_dims* dims, const void* q, const void* k,
                                      const void* v, const pka_cache* cache, const void* o,
                                      const float* lse, const void* d_o, void* dq, void* dk,
                                      void* dv, float* delta, pka_stream_t stream) {
  g_last_error[0] = 0;
  pka_status st;
  if ((st = check_dims(dims)) != PKA_OK) return st;
  const size_t need = pka_bwd_workspace_bytes(dims);
  if (need > kScratchBytes)
    return fail(PKA_ERR_WORKSPACE,
                "chunk_attn_bwd_noalloc: this shape needs %zu workspace bytes, above the "
                "library's fixed %zu (use pka_chunk_attn_bwd with a caller workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != PKA_OK) return st;
  // Same validation, plan and kernels as the call with a caller workspace. Nothing in
  // the workspace needs to start at zero: every byte the kernels read (delta, split
  // partials) is written earlier in the same call.
  return pka_chunk_attn_bwd(dims, q, k, v, cache, o, lse, d_o, dq, dk, dv, delta, ws,
                            kScratchBytes, stream);
}

static pka_status check_horizon(const pka_dims* dims, int64_t horizon) {
  if (horizon < 0 || horizon > dims->prefix_len)
    return fail(PKA_ERR_DIMS, "horizon %lld outside [0, prefix_len = %lld]", (long long)horizon,
                (long long)dims->prefix_len);
  if ((int64_t)dims->batch * dims->n_heads_kv * horizon > kMaxSeq)
    return fail(PKA_ERR_DIMS, "batch * n_heads_kv * horizon exceeds 2^31 - 1");
  return PKA_OK;
}

size_t pka_prefix_kv_grad_workspace_bytes(const pka_dims* dims, int64_t horizon) {
  if (check_dims(dims) != PKA_OK || check_horizon(dims, horizon) != PKA_OK) return 0;
  const Plan pl = plan_prefix_kv(*dims, horizon);
  if (pl.n_dkv_split <= 1) return 0;
  return align256((size_t)pl.n_dkv_split * 2 * dims->batch * dims->n_heads_kv * horizon *
                  dims->head_dim * 4);
}

pka_status pka_prefix_kv_grad(const pka_dims* dims, int64_t horizon, const void* q,
                              const pka_cache* cache, const float* lse, const void* d_o,
                              const float* delta, float* dk_prefix, float* dv_prefix,
                              void* ws, size_t ws_bytes, pka_stream_t stream) {
  g_last_error[0] = 0;
  pka_status st;
  if ((st = check_dims(dims)) != PKA_OK) return st;
  if ((st = check_group_rows(dims)) != PKA_OK) return st;
  if ((st = check_horizon(dims, horizon)) != PKA_OK) return st;
  if ((st = check_ptrs({q, lse, d_o, delta, dk_prefix, dv_prefix},
                       "q, lse, d_o, delta, dk_prefix, dv_prefix")) != PKA_OK)
    return st;
  if ((st = check_cache(cache, dims, dims->prefix_len, false)) != PKA_OK) return st;
  const size_t need = pka_prefix_kv_grad_workspace_bytes(dims, horizon);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(PKA_ERR_WORKSPACE, "prefix gradient needs %zu workspace bytes, got %zu", need,
                  ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(PKA_ERR_ALIGN, "workspace not 16-byte aligned");
  }
  if (horizon == 0) return PKA_OK;   // nothing to write
  BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.cache = cache_ref(cache);
  p.lse = lse;
  p.d_o = static_cast<const uint16_t*>(d_o);
  p.delta = const_cast<float*>(delta);
  p.dkp = dk_prefix;
  p.dvp = dv_prefix;
  p.horizon = horizon;
  p.B = dims->batch;
  p.Hq = dims->n_heads_q;
  p.Hkv = dims->n_heads_kv;
  p.G = dims->n_heads_q / dims->n_heads_kv;
  p.P = dims->prefix_len;
  p.plens = dims->prefix_lens;
  p.C = dims->chunk_len;
  p.scale = dims->softmax_scale;
  p.scale_log2 = (float)((double)dims->softmax_scale * 1.4426950408889634);
  p.plan = plan_prefix_kv(*dims, horizon);
  if (p.plan.n_dkv_split > 1) p.ws_dkv = static_cast<float*>(ws);
  hipError_t e =
      launch_prefix_kv(p, dims->head_dim, cache->type, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefix_kv_grad launch");
  return PKA_OK;
}

static pka_status append_common(const pka_dims* dims, const void* k, const void* v,
                                const pka_cache* cache, pka_stream_t stream, int want_type) {
  g_last_error[0] = 0;
  pka_status st;
  if (!dims) return fail(PKA_ERR_NULL, "dims is NULL");
  if (dims->batch < 1 || dims->n_heads_kv < 1)
    return fail(PKA_ERR_DIMS, "batch and n_heads_kv must be >= 1");
  if (dims->head_dim != 64 && dims->head_dim != 128)
    return fail(PKA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", dims->head_dim);
  if (dims->prefix_len < 0 || dims->chunk_len < 1)
    return fail(PKA_ERR_DIMS, "prefix_len must be >= 0 and chunk_len >= 1");
  if (dims->prefix_len > kMaxSeq - dims->chunk_len)
    return fail(PKA_ERR_DIMS, "prefix_len + chunk_len exceeds 2^31 - 1");
  if ((reinterpret_cast<uintptr_t>(dims->prefix_lens) & 3u) != 0)
    return fail(PKA_ERR_ALIGN, "prefix_lens not 4-byte aligned");
  if ((st = check_ptrs({k, v}, "k, v")) != PKA_OK) return st;
  if ((st = check_cache(cache, dims, dims->prefix_len + dims->chunk_len, true)) != PKA_OK) return st;
  if (cache->type != want_type)
    return fail(PKA_ERR_UNSUPPORTED, "cache type %d does not match this append (%d)", cache->type,
                want_type);
  AppendParams p{};
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.ck = cache->k;
  p.cv = cache->v;
  p.cks = static_cast<uint16_t*>(cache->k_scale);
  p.cvs = static_cast<uint16_t*>(cache->v_scale);
  p.rows = (int64_t)dims->batch * dims->n_heads_kv * dims->chunk_len;
  p.C = dims->chunk_len;
  p.P = dims->prefix_len;
  p.plens = dims->prefix_lens;
  p.cap = cache->capacity;
  p.Hkv = dims->n_heads_kv;
  p.D = dims->head_dim;
  hipError_t e = launch_append(p, want_type, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  return PKA_OK;
}

pka_status pka_kv_append_q8_0(const pka_dims* dims, const void* k, const void* v,
                              const pka_cache* cache, pka_stream_t stream) {
  return append_common(dims, k, v, cache, stream, PKA_CACHE_Q8_0);
}
pka_status pka_kv_append_f16(const pka_dims* dims, const void* k, const void* v,
                             const pka_cache* cache, pka_stream_t stream) {
  return append_common(dims, k, v, cache, stream, PKA_CACHE_F16);
}
pka_status pka_kv_append_bf16(const pka_dims* dims, const void* k, const void* v,
                              const pka_cache* cache, pka_stream_t stream) {
  return append_common(dims, k, v, cache, stream, PKA_CACHE_BF16);
}

pka_status pka_kv_dequant_q8_0(const pka_cache* cache, int32_t batch, int32_t n_heads_kv,
                               int64_t row0, int64_t rows, float* out_f32, void* out_bf16,
                               pka_stream_t stream) {
  g_last_error[0] = 0;
  if (!cache) return fail(PKA_ERR_NULL, "cache is NULL");
  if (cache->type != PKA_CACHE_Q8_0) return fail(PKA_ERR_UNSUPPORTED, "cache is not q8_0");
  if (cache->head_dim != 64 && cache->head_dim != 128)
    return fail(PKA_ERR_UNSUPPORTED, "head_dim %d not supported", cache->head_dim);
  if (batch < 1 || n_heads_kv < 1 || row0 < 0 || rows < 1)
    return fail(PKA_ERR_DIMS, "batch, n_heads_kv, rows must be >= 1 and row0 >= 0");
  if (row0 > cache->capacity - rows)
    return fail(PKA_ERR_CAPACITY, "rows [%lld, %lld) exceed capacity %lld", (long long)row0,
                (long long)(row0 + rows), (long long)cache->capacity);
  pka_status st;
  if ((st = check_ptrs({cache->k, cache->v, cache->k_scale, cache->v_scale, out_f32},
                       "cache k, v, scales, out_f32")) != PKA_OK)
    return st;
  if (out_bf16 && !aligned16(out_bf16)) return fail(PKA_ERR_ALIGN, "out_bf16 not 16-byte aligned");
  DequantParams p{};
  p.ck = static_cast<const int8_t*>(cache->k);
  p.cv = static_cast<const int8_t*>(cache->v);
  p.cks = static_cast<const uint16_t*>(cache->k_scale);
  p.cvs = static_cast<const uint16_t*>(cache->v_scale);
  p.out_f32 = out_f32;
  p.out_bf16 = static_cast<uint16_t*>(out_bf16);
  p.BH = (int64_t)batch * n_heads_kv;
  p.row0 = row0;
  p.rows = rows;
  p.cap = cache->capacity;
  p.D = cache->head_dim;
  hipError_t e = launch_dequant(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv_dequant_q8_0 launch");
  return PKA_OK;
}

static pka_status check_rs_dims(const pka_rs_dims* dims) {
  if (!dims) return fail(PKA_ERR_NULL, "dims is NULL");
  const int64_t N = dims->n_rows, K = dims->n_keep;
  const int32_t fin = dims->in_features, fout = dims->out_features;
  if (N < 1 || K < 0 || K > N)
    return fail(PKA_ERR_DIMS, "need n_rows >= 1 and 0 <= n_keep <= n_rows (got %lld, %lld)",
                (long long)N, (long long)K);
  if (fin < kRsTile || fout < kRsTile || fin % kRsTile != 0 || fout % kRsTile != 0)
    return fail(PKA_ERR_UNSUPPORTED, "in_features (%d) and out_features (%d) must be "
                "positive multiples of %d", fin, fout, kRsTile);
  if (N > kMaxSeq || (int64_t)(fin / kRsTile) * ((K + kRsTile - 1) / kRsTile) > kMaxSeq ||
      (int64_t)(fin / kRsTile) * (fout / kRsTile) > kMaxSeq || (N * (fin / 8) + 255) / 256 > kMaxSeq)
    return fail(PKA_ERR_DIMS, "row-sparse problem too large for one launch");
  return PKA_OK;
}

size_t pka_row_sparse_linear_bwd_workspace_bytes(const pka_rs_dims* dims) {
  if (check_rs_dims(dims) != PKA_OK) return 0;
  const int split = row_sparse_dx_split(dims->n_keep, dims->in_features, dims->out_features);
  if (split <= 1) return 0;
  return align256((size_t)split * dims->n_keep * dims->in_features * 4);
}

pka_status pka_row_sparse_linear_bwd(const pka_rs_dims* dims, const void* x, const void* w,
                                     const void* dy, const int32_t* keep, float* dw, void* dx,
                                     void* ws, size_t ws_bytes, pka_stream_t stream) {
  g_last_error[0] = 0;
  pka_status st;
  if ((st = check_rs_dims(dims)) != PKA_OK) return st;
  const int64_t N = dims->n_rows, K = dims->n_keep;
  const int32_t fin = dims->in_features, fout = dims->out_features;
  if (!dw && !dx) return PKA_OK;
  if ((st = check_ptrs({dy}, "dy")) != PKA_OK) return st;
  if (dw && (st = check_ptrs({x, dw}, "x, dw")) != PKA_OK) return st;
  if (dx && (st = check_ptrs({w, dx}, "w, dx")) != PKA_OK) return st;
  if (K > 0 && !keep) return fail(PKA_ERR_NULL, "keep is NULL");
  if ((reinterpret_cast<uintptr_t>(keep) & 3u) != 0)
    return fail(PKA_ERR_ALIGN, "keep not 4-byte aligned");
  const int split = dx ? row_sparse_dx_split(K, fin, fout) : 1;
  if (split > 1) {
    const size_t need = pka_row_sparse_linear_bwd_workspace_bytes(dims);
    if (!ws || ws_bytes < need)
      return fail(PKA_ERR_WORKSPACE, "row-sparse dX needs %zu workspace bytes, got %zu", need,
                  ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(PKA_ERR_ALIGN, "workspace not 16-byte aligned");
  }
  RsParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.w = static_cast<const uint16_t*>(w);
  p.dy = static_cast<const uint16_t*>(dy);
  p.keep = keep;
  p.dw = dw;
  p.dx = static_cast<uint16_t*>(dx);
  p.N = N;
  p.K = K;
  p.in = fin;
  p.out = fout;
  p.dx_split = split;
  p.ws = split > 1 ? static_cast<float*>(ws) : nullptr;
  hipError_t e = launch_row_sparse_bwd(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "row_sparse_linear_bwd launch");
  return PKA_OK;
}

pka_status pka_profile_enable(int32_t on) {
  g_prof_on.store(on != 0);
  return PKA_OK;
}

pka_status pka_profile_select(uint32_t kernel_mask) {
  g_prof_mask.store(kernel_mask);
  return PKA_OK;
}

pka_status pka_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& sl : g_prof) {
    sl.used = 0;
    sl.dropped = 0;
    sl.open = false;
  }
  return PKA_OK;
}

pka_status pka_profile_read(int32_t kernel, double* total_ms, int64_t* launches,
                            int64_t* dropped) {
  g_last_error[0] = 0;
  if (kernel < 0 || kernel >= PKA_KERNEL_COUNT)
    return fail(PKA_ERR_DIMS, "unknown kernel id %d", kernel);
  if (!total_ms || !launches) return fail(PKA_ERR_NULL, "total_ms / launches is NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfSlot& sl = g_prof[kernel];
  double sum = 0.0;
  for (int64_t i = 0; i < sl.used; ++i) {
    hipError_t e = hipEventSynchronize(sl.end[i]);
    if (e != hipSuccess) return hip_fail(e, "profile event sync");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, sl.begin[i], sl.end[i]);
    if (e != hipSuccess) return hip_fail(e, "profile elapsed time");
    sum += ms;
  }
  *total_ms = sum;
  *launches = sl.used;
  if (dropped) *dropped = sl.dropped;
  return PKA_OK;
}

}  // extern "C"
