// Row-sparse linear backward: parameters and launcher shared by the host layer and
// row_sparse.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pka {

struct RsParams {
  const uint16_t* x;     // bf16 [N][in]
  const uint16_t* w;     // bf16 [out][in]
  const uint16_t* dy;    // bf16 [N][out]
  const int32_t* keep;   // int32 [K], kept row indices (strictly increasing, in [0, N))
  float* dw;             // f32 [out][in], or null (not computed)
  uint16_t* dx;          // bf16 [N][in], or null (not computed)
  int64_t N, K;
  int in, out;
};

// Workgroup tile of both products (output rows x columns) and its k-stage.
constexpr int kRsTile = 128;
constexpr int kRsStage = 64;

hipError_t launch_row_sparse_bwd(const RsParams& p, hipStream_t s);

}  // namespace pka
