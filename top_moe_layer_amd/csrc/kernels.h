// Host launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace topmoe {

enum GemmKind {
  KIND_GATEUP = 0,      // h = SiLU(A Wg^T) * (A Wu^T), rows gathered from x
  KIND_DOWN_Y = 1,      // y[token] = alpha * (h Wd^T), written in the output dtype
  KIND_DOWN_SLOTS = 2,  // slot[entry] = alpha * (h Wd^T), float32
};

struct GemmParams {
  const void* A;           // gate/up: x [N, K]; down: h [rows, K] (grouped row order)
  const void* B0;          // gate/up: Wg [E, Nout, K]; down: Wd [E, Nout, K]
  const void* B1;          // gate/up: Wu [E, Nout, K]; down: unused
  void* out;               // gate/up: h [rows, Nout]; down: y [N, Nout] or slots [rows, Nout]
  const int32_t* entries;  // grouped row -> entry id t*k + j; NULL = identity (dense)
  const int32_t* offsets;  // [E+1] group row offsets; NULL = one group of M rows
  const float* alpha;      // [rows] weight of each grouped row (down); NULL = 1
  int64_t M;               // rows when offsets == NULL
  int E, k;
  int Nout, K;
};

enum RouterMode {
  ROUTER_MODE_LDS = 0,    // W_router staged in LDS, one token per wavefront
  ROUTER_MODE_SPLIT = 1,  // one token per block, H split over the wavefronts
};

hipError_t launch_router(const void* x, const float* Wr, int dtype, int64_t N, int H, int E,
                         int k, int tb, int nblk, int mode, int32_t* topk_idx, float* alpha,
                         int32_t* count_part, float* psum_part, hipStream_t s);

hipError_t launch_permute(const int32_t* count_part, const float* psum_part,
                          const int32_t* topk_idx, const float* alpha, int nblk, int E, int k,
                          int tb, int64_t N, float coef, int32_t* offsets, float* aux,
                          int32_t* sorted_entry, float* alpha_g, int32_t* sorted_tok,
                          hipStream_t s);

hipError_t launch_combine(const float* slots, const int32_t* topk_idx, int64_t N, int H, int k,
                          int dtype, void* y, hipStream_t s);

hipError_t launch_empty_route(int E, int32_t* offsets, float* aux, hipStream_t s);

hipError_t launch_gemm(int kind, int dtype, GemmShape shape, const GemmParams& p,
                       int64_t mtiles, hipStream_t s);

}  // namespace topmoe
