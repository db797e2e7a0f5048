// Tile-height-aware entry points of the FP8 MFMA kernel (k_f8.hip).  The
// kernel runs 256-row tiles (bn = 256 or 192) or 128-row tiles with bn = 192;
// the forms in common.h without bm mean bm = 256.
#pragma once
#include "common.h"

namespace mgemm {
bool f8_mfma_supports_bm(const Problem& p, int bn, int bm);
// K ranges a request turns into for bn x bm tiles (0 when the partials do
// not fit the workspace).
int f8_splits_bm(const Problem& p, int bn, int bm, int requested, const Workspace& ws);
hipError_t launch_f8_gemm_bm(const Problem& p, const float* sa, const float* sb, int bn, int bm,
                             int ksplit, const Workspace& ws, hipStream_t s);
}  // namespace mgemm
