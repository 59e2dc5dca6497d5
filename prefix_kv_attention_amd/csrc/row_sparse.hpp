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
  const int32_t* keep;   // int32 [K], distinct kept row indices, any order (entries
                         // outside [0, N) are skipped)
  float* dw;             // f32 [out][in], or null (not computed)
  uint16_t* dx;          // bf16 [N][in], or null (not computed)
  float* ws;             // dX split over output features: f32 partials [dx_split][K][in]
  int64_t N, K;
  int in, out;
  int dx_split;          // 1: dX written directly; > 1: partials, then a reduction
};

// Workgroup tile of both products (output rows x columns) and its k-stage.
constexpr int kRsTile = 128;
constexpr int kRsStage = 64;

// Splits of the dX product over its contraction (output features) so that a grid of
// few tiles still fills the CUs: (256 / tiles), at most 8, each split at least 4
// k-stages; 1 when the tiles alone reach 256.
int row_sparse_dx_split(int64_t n_keep, int in_features, int out_features);

hipError_t launch_row_sparse_bwd(const RsParams& p, hipStream_t s);

}  // namespace pka
