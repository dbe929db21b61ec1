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

struct GemmParams {
  const void* A;           // gate/up, bwd gu: x [N, K]; bwd dh: dy [N, K];
                           // down: h or [dg|du] [rows, K];
                           // wgrad: [M, ldk] transposed activations (padded group columns)
  const void* A1;          // wgrad pair: second A [M, ldk]
  const void* B0;          // gate/up, bwd gu: Wg [E, Nout, K]; bwd dh: Wd^T [E, Nout, K];
                           // down: Wd or [Wg|Wu]^T [E, Nout, K]; wgrad: [Nout, ldk]
  const void* B1;          // gate/up, bwd gu: Wu [E, Nout, K]
  const void* B2;          // (a third B operand; unused by the current kinds)
  const void* gu;          // bwd dh: the pairs (g, u) [rows, Nout] written by bwd gu
  void* out;               // gate/up: h [rows, Nout]; down: y [N, Nout] or slots [rows, Nout];
                           // bwd gu: pairs (g, u) [rows, Nout]; bwd dh: [dg | du] [rows, 2 Nout];
                           // wgrad: [groups, M, Nout]
  void* out1;              // bwd gu: h^T; bwd dh: dg^T [Nout, ldk];
                           // wgrad pair: second [groups, M, Nout]
  void* out2;              // bwd dh: du^T [Nout, ldk]; bwd gu: NULL, or h [rows, Nout] row-major
                           // (the training forward, which keeps g, u for the backward)
  void* out3;              // (unused)
  float* dalpha_part;      // bwd dh: [entries, ceil(Nout / BN)] partial dh_raw . h; NULL = skip
  const int32_t* entries;  // grouped row -> entry id t*k + j; NULL = identity (dense)
  const int32_t* offsets;  // [E+1] group row offsets; NULL = one group of M rows
                           // (wgrad: of kcount rows)
  const float* alpha;      // [rows] weight of each grouped row (down, bwd h); NULL = 1
  const void* residual;    // down into y: [N, Nout] added before rounding; NULL = none
  int64_t M;               // rows when offsets == NULL (wgrad: output rows per group)
  int64_t ldk;             // bwd h / wgrad: row length of the padded-column matrices
  int64_t kcount;          // wgrad with offsets == NULL: rows of the single group
  int E, k;
  int Nout, K;
  // down projections: the K slices split into ksplit chunks of kchunk slices
  // (ksplit <= 1: none); chunk c of a tile writes its raw fp32 accumulators
  // to partial [ksplit, M, Nout] (grouped rows) and launch_splitk_reduce
  // applies the epilogue to their sum
  int ksplit, kchunk;
  float* partial;
  // In-block routing (few entries, forward kinds with 64-row tiles): when
  // inl_topk is not NULL, every block groups the inl_n = N * k entries of
  // inl_topk [N, k] (and their weights inl_alpha) by expert itself -- the
  // expert offsets, the stable order of entries within an expert, the rows'
  // alpha -- instead of reading offsets / entries / alpha.  With
  // inl_outputs the launch has one block more, the last, which takes no
  // tile and writes the routing outputs that the permutation kernel would
  // have: inl_offsets_out [E+1] and inl_sorted_out [N*k] (each when not
  // NULL), and aux / z-loss from the router's per-block partials
  // (inl_psum_part [E, inl_nblk], inl_z_part [inl_nblk]) into inl_aux_out /
  // inl_z_out (each when not NULL).
  const int32_t* inl_topk;
  const float* inl_alpha;
  int inl_n, inl_nblk, inl_outputs;
  int32_t* inl_offsets_out;
  int32_t* inl_sorted_out;
  const float* inl_psum_part;
  const float* inl_z_part;
  float* inl_aux_out;
  float* inl_z_out;
  float inl_coef, inl_z_coef;
  int64_t inl_tokens;
  // Every token against every expert (decode-sized calls, gate/up): with
  // allx_n = N > 0 the groups are the E experts, each of the N rows of A in
  // order (group e's row t is A row t, written to out row e * N + t); the
  // down projection, with in-block routing, then reads entry (t, j) of
  // expert e from A row e * N + t.
  int64_t allx_n;
  // Router blocks riding on a gate/up launch (rt_blocks > 0, E <= 16): the
  // last rt_blocks blocks route tokens [b * rt_tb, b * rt_tb + rt_tb) of A
  // against rt_wr [E, K] exactly as the split router kernel does, writing
  // rt_topk / rt_alpha [N, k] and the per-block partials rt_count /
  // rt_psum [E, rt_blocks] and rt_zpart [rt_blocks].
  const float* rt_wr;
  int rt_blocks, rt_tb, rt_renorm;
  int64_t rt_n;
  int32_t* rt_topk;
  float* rt_alpha;
  int32_t* rt_count;
  float* rt_psum;
  float* rt_zpart;
};

enum RouterMode {
  ROUTER_MODE_LDS = 0,    // W_router staged in LDS, 16 tokens per wavefront pass
  ROUTER_MODE_SPLIT = 1,  // one token per block, H split over the wavefronts
  ROUTER_MODE_LDS16 = 2,  // as LDS, 16 lanes per token: four wavefronts per block
};

// probs [N, E] and lse [N] (logsumexp of the logits) are optional outputs for
// the backward; z_part [blocks] always receives each block's sum of lse^2.
hipError_t launch_router(const void* x, const float* Wr, int dtype, int64_t N, int H, int E,
                         int k, bool renorm, int tb, int nblk, int mode, int32_t* topk_idx,
                         float* alpha, float* probs, float* lse,
                         int32_t* count_part, float* psum_part, float* z_part, const Launch& s);

// cap <= 0: no expert capacity.  offsets: of the kept entries; counts_off
// (optional): of every selection.  keep [N*k] (optional): 1 where the entry is kept.
// topk_copy / alpha_copy [N*k] and offsets_copy [E+1] (optional): second
// copies of topk_idx, alpha and offsets (the training forward keeps the
// routing for the backward besides the caller's outputs).
hipError_t launch_permute(const int32_t* count_part, const float* psum_part,
                          const float* z_part, const int32_t* topk_idx, const float* alpha,
                          int nblk, int E, int k, int tb, int64_t N, float coef, float z_coef,
                          int cap, int32_t* offsets, int32_t* counts_off, float* aux,
                          float* z_loss, int32_t* sorted_entry, float* alpha_g,
                          int32_t* sorted_tok, uint8_t* keep, int32_t* topk_copy,
                          float* alpha_copy, int32_t* offsets_copy, const Launch& s);

hipError_t launch_combine(const void* slots, const int32_t* topk_idx, const uint8_t* keep,
                          const void* residual, int64_t N, int H, int k, int dtype, void* y,
                          const Launch& s);

hipError_t launch_empty_route(int E, int32_t* offsets, float* aux, float* z_loss,
                              const Launch& s);

// The down projection's epilogue over split-K partial sums: for each grouped
// row r < (offsets ? offsets[E] : M) and column c, s = sum over the ksplit
// chunks in order of partial[chunk][r][c]; then y[entry / k][c] =
// (residual) + alpha[r] * s rounded once (slots == false) or
// out[entry][c] = alpha[r] * s in the dtype (slots == true); entries / alpha
// NULL = identity / 1.
hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int Nout,
                                const int32_t* offsets, int E, const int32_t* entries,
                                const float* alpha, int k, const void* residual, int dtype,
                                bool slots, void* out, const Launch& s);

hipError_t launch_gemm(int kind, int dtype, GemmShape shape, const GemmParams& p,
                       int64_t mtiles, const Launch& s);

// ---- backward
// out[b][c][col0 + r] = src[b][r][c]; R, C multiples of 64.
struct TransposeJob {
  const void* src;
  void* dst;
  int R, C, batch, col0;
  int64_t ldo, src_bs, dst_bs;  // out row pitch; per-batch element strides
};
struct TransposeJobs {
  TransposeJob job[3];
  int n;
};
// Gathered transpose into padded group columns (see backward.hip).
struct GatherTransposeJob {
  const void* src;      // [*, C]
  void* dst;            // [C, ldo]
  const float* scale;   // per grouped row, or NULL
};
struct GatherTransposeJobs {
  GatherTransposeJob job[2];
  int n;
  const int32_t* offsets;  // [E+1] group offsets, or NULL: one group of `rows`
  const int32_t* entries;  // grouped row -> entry id (source row entries / k), or NULL
  int E, k, C;
  int64_t rows, ldo;
};

hipError_t launch_transpose(int dtype, const TransposeJobs& jobs, int max_tiles, int max_batch,
                            const Launch& s);
hipError_t launch_gather_transpose(int dtype, const GatherTransposeJobs& jobs, int64_t ldo,
                                   const Launch& s);
// counts_off [E+1]: exclusive prefix sums of every expert's selections (before
// any capacity); keep / lse as from the routing (NULL: all kept / no z-loss).
hipError_t launch_router_bwd(const float* probs, const int32_t* topk_idx,
                             const float* dalpha_part, int nt, const int32_t* counts_off,
                             const uint8_t* keep, const float* lse, int64_t N, int E, int k,
                             bool renorm, float aux_scale, const float* aux_mul,
                             float z_scale, const float* z_mul, float* dr, const Launch& s);
hipError_t launch_combine_bwd(const void* slots, const int32_t* topk_idx, const uint8_t* keep,
                              const float* dr, const float* Wr, int64_t N, int H, int E, int k,
                              int dtype, void* dx, const Launch& s);
int dwr_chunks(int64_t N);
hipError_t launch_dwr(const void* x, const float* dr, int64_t N, int H, int E, int dtype,
                      float* part, float* dWr, const Launch& s);

}  // namespace topmoe
