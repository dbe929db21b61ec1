// Host launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <tuple>

#include "plan.h"

namespace topmoe {

// Where a launcher enqueues its kernel: the stream and, for stage timing,
// optional events that the dispatch itself timestamps at the kernel's start
// and end (hipExtLaunchKernel), so they bracket exactly the kernel's
// execution.  `launched` tells the caller whether a kernel consumed them.
struct Launch {
  hipStream_t s = nullptr;
  hipEvent_t start = nullptr, stop = nullptr;
  mutable bool launched = false;
};

template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, unsigned shm,
                         const Launch& L, A... a) {
  L.launched = true;
  if (L.start == nullptr && L.stop == nullptr) {
    hipLaunchKernelGGL(kernel, grid, block, shm, L.s, a...);
    return hipGetLastError();
  }
  std::tuple<P...> args{P(a)...};
  void* ptrs[sizeof...(P)];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, args);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shm, L.s,
                            L.start, L.stop, 0);
}

enum GemmKind {
  KIND_GATEUP = 0,      // h = SiLU(A Wg^T) * (A Wu^T), rows gathered from x
  KIND_DOWN_Y = 1,      // y[token] = alpha * (h Wd^T), written in the output dtype
  KIND_DOWN_SLOTS = 2,  // slot[entry] = alpha * (h Wd^T), in the operand dtype
};

struct GemmParams {
  const void* A;           // gate/up: x [N, K]; down: h [rows, K] (grouped row order)
  const void* B0;          // gate/up: Wg [E, Nout, K]; down: Wd [E, Nout, K]
  const void* B1;          // gate/up: Wu [E, Nout, K]; down: unused
  void* out;               // gate/up: h [rows, Nout]; down: y [N, Nout] or slots [rows, Nout]
  const int32_t* entries;  // grouped row -> entry id t*k + j; NULL = identity (dense)
  const int32_t* offsets;  // [E+1] group row offsets; NULL = one group of M rows
  const float* alpha;      // [rows] weight of each grouped row (down); NULL = 1
  const void* residual;    // down into y: [N, Nout] added before rounding; NULL = none
  int64_t M;               // rows when offsets == NULL
  int E, k;
  int Nout, K;
};

enum RouterMode {
  ROUTER_MODE_LDS = 0,    // W_router staged in LDS, one token per wavefront
  ROUTER_MODE_SPLIT = 1,  // one token per block, H split over the wavefronts
};

hipError_t launch_router(const void* x, const float* Wr, int dtype, int64_t N, int H, int E,
                         int k, bool renorm, int tb, int nblk, int mode, int32_t* topk_idx,
                         float* alpha,
                         int32_t* count_part, float* psum_part, const Launch& s);

hipError_t launch_permute(const int32_t* count_part, const float* psum_part,
                          const int32_t* topk_idx, const float* alpha, int nblk, int E, int k,
                          int tb, int64_t N, float coef, int32_t* offsets, float* aux,
                          int32_t* sorted_entry, float* alpha_g, int32_t* sorted_tok,
                          const Launch& s);

hipError_t launch_combine(const void* slots, const int32_t* topk_idx, const void* residual,
                          int64_t N, int H, int k, int dtype, void* y, const Launch& s);

hipError_t launch_empty_route(int E, int32_t* offsets, float* aux, const Launch& s);

hipError_t launch_gemm(int kind, int dtype, GemmShape shape, const GemmParams& p,
                       int64_t mtiles, const Launch& s);

}  // namespace topmoe
