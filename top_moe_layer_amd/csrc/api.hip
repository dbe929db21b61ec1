// C ABI entry points: validate on the host, carve the workspace, enqueue the
// kernels.  See include/topmoe.h for the contract of every function.
#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "plan.h"

#include "../../include/topmoe.h"

namespace topmoe {
hipError_t launch_gemm_bf16(int kind, GemmShape sh, const GemmParams& p, int64_t mtiles,
                            const Launch& s);
hipError_t launch_gemm_f32(int kind, GemmShape sh, const GemmParams& p, int64_t mtiles,
                           const Launch& s);

hipError_t launch_gemm(int kind, int dtype, GemmShape shape, const GemmParams& p,
                       int64_t mtiles, const Launch& s) {
  return dtype == TOPMOE_DTYPE_FP32 ? launch_gemm_f32(kind, shape, p, mtiles, s)
                                    : launch_gemm_bf16(kind, shape, p, mtiles, s);
}
}  // namespace topmoe

using namespace topmoe;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Stage i's launch: the stream plus, when timing is requested, events
// 2i / 2i+1 stamped by the stage's kernel dispatch.
struct Stages {
  void* const* ev;
  hipStream_t s;
  Launch at(int i) const {
    Launch L;
    L.s = s;
    if (ev) {
      L.start = static_cast<hipEvent_t>(ev[2 * i]);
      L.stop = static_cast<hipEvent_t>(ev[2 * i + 1]);
    }
    return L;
  }
  // A stage that enqueued no kernel still gets both events (zero length).
  hipError_t close(const Launch& L) const {
    if (!ev || L.launched) return hipSuccess;
    const hipError_t e = hipEventRecord(L.start, s);
    return e != hipSuccess ? e : hipEventRecord(L.stop, s);
  }
};

#define TOPMOE_TRY(expr)                              \
  do {                                                \
    if ((expr) != hipSuccess) return TOPMOE_ERR_HIP;  \
  } while (0)

}  // namespace

extern "C" {

int topmoe_version(void) { return 110; }

const char* topmoe_strerror(int status) {
  switch (status) {
    case TOPMOE_OK: return "ok";
    case TOPMOE_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case TOPMOE_ERR_BAD_SHAPE:
      return "shape outside the supported limits (H, I multiples of 64; 1 <= E <= 64; "
             "1 <= k <= E; N >= 0; sizes within 32-bit row ids)";
    case TOPMOE_ERR_UNSUPPORTED_DTYPE: return "dtype must be TOPMOE_DTYPE_FP32 or TOPMOE_DTYPE_BF16";
    case TOPMOE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the *_workspace_bytes() size";
    case TOPMOE_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case TOPMOE_ERR_BAD_ARG:
      return "invalid argument (aux_coef negative or not finite, unknown flag bits, or a "
             "misaligned pointer)";
  }
  return "unknown status";
}

size_t ffn_workspace_bytes(int64_t N, int64_t H, int64_t I, int dtype) {
  FfnPlan pl;
  return plan_ffn(N, H, I, dtype, &pl) == TOPMOE_OK ? pl.total : 0;
}

size_t moe_workspace_bytes(int64_t N, int64_t H, int64_t I, int E, int k, int dtype) {
  MoePlan pl;
  return plan_moe(N, H, I, E, k, dtype, &pl) == TOPMOE_OK ? pl.total : 0;
}

int ffn_swiglu_fwd(const void* x, const void* Wg, const void* Wu, const void* Wd,
                   const void* residual, void* y, int64_t N, int64_t H, int64_t I, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream,
                   void* const* stage_events) {
  FfnPlan pl;
  const int status = plan_ffn(N, H, I, dtype, &pl);
  if (status != TOPMOE_OK) return status;
  // zero-size tensors (N == 0) are never touched and may be NULL
  if (!Wg || !Wu || !Wd || !workspace || (N > 0 && (!x || !y))) return TOPMOE_ERR_NULL_ARG;
  if (workspace_bytes < pl.total) return TOPMOE_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(x, 16) || !aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) ||
      !aligned(residual, 16) || !aligned(y, 16) || !aligned(workspace, 256))
    return TOPMOE_ERR_BAD_ARG;

  const Stages st{stage_events, static_cast<hipStream_t>(stream)};
  char* ws = static_cast<char*>(workspace);
  void* h = ws + pl.off_h;

  const Launch l0 = st.at(0);
  if (N > 0) {
    GemmParams up{};
    up.A = x; up.B0 = Wg; up.B1 = Wu; up.out = h;
    up.entries = nullptr; up.offsets = nullptr; up.alpha = nullptr;
    up.M = N; up.E = 1; up.k = 1; up.Nout = int(I); up.K = int(H);
    TOPMOE_TRY(launch_gemm(KIND_GATEUP, dtype, pl.up, up, (N + pl.up.bm - 1) / pl.up.bm, l0));
  }
  TOPMOE_TRY(st.close(l0));
  const Launch l1 = st.at(1);
  if (N > 0) {
    GemmParams dn{};
    dn.A = h; dn.B0 = Wd; dn.B1 = nullptr; dn.out = y; dn.residual = residual;
    dn.entries = nullptr; dn.offsets = nullptr; dn.alpha = nullptr;
    dn.M = N; dn.E = 1; dn.k = 1; dn.Nout = int(H); dn.K = int(I);
    TOPMOE_TRY(launch_gemm(KIND_DOWN_Y, dtype, pl.down, dn, (N + pl.down.bm - 1) / pl.down.bm, l1));
  }
  TOPMOE_TRY(st.close(l1));
  return TOPMOE_OK;
}

int moe_ffn_fwd(const void* x, const float* Wr, const void* Wg, const void* Wu, const void* Wd,
                const void* residual, int64_t N, int64_t H, int64_t I, int E, int k,
                float aux_coef, int flags, int dtype,
                void* y, int32_t* topk_idx, float* alpha, float* aux_loss,
                int32_t* expert_offsets, int32_t* sorted_token_ids, void* workspace,
                size_t workspace_bytes, void* stream, void* const* stage_events) {
  MoePlan pl;
  const int status = plan_moe(N, H, I, E, k, dtype, &pl);
  if (status != TOPMOE_OK) return status;
  // zero-size tensors (N == 0) are never touched and may be NULL
  if (!Wr || !Wg || !Wu || !Wd || !aux_loss || !workspace ||
      (N > 0 && (!x || !y || !topk_idx || !alpha)))
    return TOPMOE_ERR_NULL_ARG;
  if (!(aux_coef >= 0.0f) || isinf(aux_coef)) return TOPMOE_ERR_BAD_ARG;
  if (flags & ~TOPMOE_MOE_RAW_TOPK_WEIGHTS) return TOPMOE_ERR_BAD_ARG;
  const bool renorm = (flags & TOPMOE_MOE_RAW_TOPK_WEIGHTS) == 0;
  if (workspace_bytes < pl.total) return TOPMOE_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(Wg, 16) || !aligned(Wu, 16) ||
      !aligned(Wd, 16) || !aligned(residual, 16) || !aligned(y, 16) || !aligned(topk_idx, 4) ||
      !aligned(alpha, 4) ||
      !aligned(aux_loss, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_token_ids, 4) ||
      !aligned(workspace, 256))
    return TOPMOE_ERR_BAD_ARG;

  const Stages st{stage_events, static_cast<hipStream_t>(stream)};
  char* ws = static_cast<char*>(workspace);
  int32_t* count_part = reinterpret_cast<int32_t*>(ws + pl.off_count_part);
  float* psum_part = reinterpret_cast<float*>(ws + pl.off_psum_part);
  int32_t* offsets = expert_offsets ? expert_offsets : reinterpret_cast<int32_t*>(ws + pl.off_offsets);
  int32_t* sorted_entry = reinterpret_cast<int32_t*>(ws + pl.off_sorted);
  float* alpha_g = reinterpret_cast<float*>(ws + pl.off_alpha_g);
  void* h = ws + pl.off_h;
  void* slots = ws + pl.off_slots;

  if (N == 0) {
    for (int i = 0; i < TOPMOE_MOE_STAGES; ++i) {
      const Launch L = st.at(i);
      if (i == 1) TOPMOE_TRY(launch_empty_route(E, offsets, aux_loss, L));
      TOPMOE_TRY(st.close(L));
    }
    return TOPMOE_OK;
  }

  // 0: router, softmax, top-k, alpha, per-block counts and sums of p
  const Launch l0 = st.at(0);
  TOPMOE_TRY(launch_router(x, Wr, dtype, N, int(H), E, k, renorm, pl.tb, pl.nblk,
                           pl.router_mode, topk_idx, alpha, count_part, psum_part, l0));
  TOPMOE_TRY(st.close(l0));
  // 1: expert offsets, aux loss, stable scatter of entries into expert groups
  const Launch l1 = st.at(1);
  TOPMOE_TRY(launch_permute(count_part, psum_part, topk_idx, alpha, pl.nblk, E, k, pl.tb, N,
                            aux_coef, offsets, aux_loss, sorted_entry, alpha_g,
                            sorted_token_ids, l1));
  TOPMOE_TRY(st.close(l1));
  // 2: grouped gate/up GEMM + SiLU * up
  const Launch l2 = st.at(2);
  GemmParams up{};
  up.A = x; up.B0 = Wg; up.B1 = Wu; up.out = h;
  up.entries = sorted_entry; up.offsets = offsets; up.alpha = nullptr;
  up.M = pl.rows; up.E = E; up.k = k; up.Nout = int(I); up.K = int(H);
  TOPMOE_TRY(launch_gemm(KIND_GATEUP, dtype, pl.up, up, pl.up_mtiles, l2));
  TOPMOE_TRY(st.close(l2));
  // 3: grouped down GEMM, alpha-scaled, into y (k == 1) or the k slots
  const Launch l3 = st.at(3);
  GemmParams dn{};
  dn.A = h; dn.B0 = Wd; dn.B1 = nullptr; dn.out = k == 1 ? y : slots;
  dn.residual = k == 1 ? residual : nullptr;  // k >= 2: added by the combine
  dn.entries = sorted_entry; dn.offsets = offsets; dn.alpha = alpha_g;
  dn.M = pl.rows; dn.E = E; dn.k = k; dn.Nout = int(H); dn.K = int(I);
  TOPMOE_TRY(launch_gemm(k == 1 ? KIND_DOWN_Y : KIND_DOWN_SLOTS, dtype, pl.down, dn,
                         pl.down_mtiles, l3));
  TOPMOE_TRY(st.close(l3));
  // 4: fixed-order combine of the k slots
  const Launch l4 = st.at(4);
  if (k >= 2) TOPMOE_TRY(launch_combine(slots, topk_idx, residual, N, int(H), k, dtype, y, l4));
  TOPMOE_TRY(st.close(l4));
  return TOPMOE_OK;
}

int topmoe_events_create(int n, void** events) {
  if (!events || n < 0) return TOPMOE_ERR_NULL_ARG;
  for (int i = 0; i < n; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return TOPMOE_ERR_HIP;
    events[i] = e;
  }
  return TOPMOE_OK;
}

int topmoe_events_destroy(int n, void** events) {
  if (!events || n < 0) return TOPMOE_ERR_NULL_ARG;
  for (int i = 0; i < n; ++i) {
    if (events[i] && hipEventDestroy(static_cast<hipEvent_t>(events[i])) != hipSuccess)
      return TOPMOE_ERR_HIP;
    events[i] = nullptr;
  }
  return TOPMOE_OK;
}

int topmoe_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return TOPMOE_ERR_NULL_ARG;
  if (hipEventSynchronize(static_cast<hipEvent_t>(stop)) != hipSuccess) return TOPMOE_ERR_HIP;
  if (hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)) !=
      hipSuccess)
    return TOPMOE_ERR_HIP;
  return TOPMOE_OK;
}

}  // extern "C"
