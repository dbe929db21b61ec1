// C ABI entry points: validate on the host, carve the workspace, enqueue the
// kernels.  See include/topmoe.h for the contract of every function.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"
#include "plan.h"

#include "../../include/topmoe.h"

namespace topmoe {
hipError_t launch_gemm_bf16(int kind, GemmShape sh, const GemmParams& p, int64_t mtiles,
                            const Launch& s);
hipError_t launch_gemm_f32(int kind, GemmShape sh, const GemmParams& p, int64_t mtiles,
                           const Launch& s);

bool gemm_shape_supported_bf16(int kind, const GemmShape& sh);
bool gemm_shape_supported_f32(int kind, const GemmShape& sh);

bool gemm_shape_supported(int kind, int dtype, const GemmShape& sh) {
  return dtype == TOPMOE_DTYPE_FP32 ? gemm_shape_supported_f32(kind, sh)
                                    : gemm_shape_supported_bf16(kind, sh);
}

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

// Expert capacity ceil(capacity_factor * N * k / E); 0 = no capacity (also
// when it could not be reached).
int capacity_of(double capacity_factor, int64_t N, int k, int E) {
  if (capacity_factor <= 0.0) return 0;
  const double c = ceil(capacity_factor * double(N) * double(k) / double(E));
  return c >= double(N) ? 0 : int(c);
}

bool nonneg_finite(float v) { return v >= 0.0f && !isinf(v); }

#define TOPMOE_TRY(expr)                              \
  do {                                                \
    if ((expr) != hipSuccess) return TOPMOE_ERR_HIP;  \
  } while (0)

}  // namespace

extern "C" {

int topmoe_version(void) { return 151; }

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
    case TOPMOE_ERR_SCRATCH_TOO_SMALL:
      return "the problem needs more workspace (moe_workspace_bytes()) than the fixed scratch "
             "of moe_ffn_fwd_noalloc (TOPMOE_NOALLOC_SCRATCH_BYTES, 64 MiB)";
    case TOPMOE_ERR_BAD_ARG:
      return "invalid argument (aux_coef, z_coef or capacity_factor negative or not finite, "
             "aux_grad or z_grad not finite, unknown flag bits, a misaligned pointer, or a "
             "launch-shape override that is not instantiated)";
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

int moe_ffn_fwd_path(int64_t N, int64_t H, int64_t I, int E, int k, float capacity_factor,
                     int dtype, int32_t* info, int n) {
  if (n > 0 && !info) return TOPMOE_ERR_NULL_ARG;
  if (!nonneg_finite(capacity_factor)) return TOPMOE_ERR_BAD_ARG;
  MoePlan pl;
  const int status = plan_moe(N, H, I, E, k, dtype, &pl);
  if (status != TOPMOE_OK) return status;
  const bool inl = capacity_of(capacity_factor, N, k, E) == 0 && pl.inline_ok;
  const int32_t v[TOPMOE_PATH_FIELDS] = {
      pl.router_mode, pl.tb, pl.nblk, pl.up.bm, pl.up.bn, pl.up.stages, pl.down.bm,
      pl.down.bn, pl.down.stages, pl.down_ksplit, inl ? 1 : 0, inl && pl.allx ? 1 : 0};
  for (int i = 0; i < n; ++i) info[i] = i < TOPMOE_PATH_FIELDS ? v[i] : -1;
  return TOPMOE_OK;
}

}  // extern "C"

namespace {

// The down projection (into y, or into the k-slots): one GEMM, or with a K
// split the GEMM's chunks into fp32 partials and the reduce that sums them in
// order and applies the epilogue (the stage's start event on the first
// launch, its stop event on the second).
hipError_t launch_down(int dtype, const GemmShape& sh, const GemmParams& p, int64_t mtiles,
                       bool slots, const Launch& L) {
  if (p.ksplit <= 1)
    return launch_gemm(slots ? KIND_DOWN_SLOTS : KIND_DOWN_Y, dtype, sh, p, mtiles, L);
  Launch first = L, second = L;
  first.stop = nullptr;
  second.start = nullptr;
  hipError_t e = launch_gemm(KIND_DOWN_PARTIAL, dtype, sh, p, mtiles, first);
  if (e != hipSuccess) return e;
  e = launch_splitk_reduce(p.partial, p.ksplit, p.M, p.Nout, p.offsets, p.E, p.entries, p.alpha,
                           p.k, slots ? nullptr : p.residual, dtype, slots, p.out, second);
  L.launched = first.launched || second.launched;
  return e;
}

// The dense forward; with `saved` (a backward workspace) the gate/up
// projection also keeps the pairs (g, u) and h^T there for
// ffn_swiglu_bwd_saved.
int ffn_fwd_impl(const void* x, const void* Wg, const void* Wu, const void* Wd,
                 const void* residual, void* y, int64_t N, int64_t H, int64_t I, int dtype,
                 void* workspace, size_t workspace_bytes, void* saved, size_t saved_bytes,
                 bool train, void* stream, void* const* stage_events) {
  FfnPlan pl;
  const int status = plan_ffn(N, H, I, dtype, &pl);
  if (status != TOPMOE_OK) return status;
  FfnBwdPlan bpl;
  if (train) {
    const int bst = plan_ffn_bwd(N, H, I, dtype, &bpl);
    if (bst != TOPMOE_OK) return bst;
    if (!saved) return TOPMOE_ERR_NULL_ARG;
    if (saved_bytes < bpl.total) return TOPMOE_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(saved, 256)) return TOPMOE_ERR_BAD_ARG;
  }
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
  if (N > 0 && train) {  // the backward's g, u projection, writing h row-major as well
    char* sv = static_cast<char*>(saved);
    GemmParams g{};
    g.A = x; g.B0 = Wg; g.B1 = Wu; g.out = sv + bpl.off_gu; g.out1 = sv + bpl.off_hT;
    g.out2 = h;
    g.M = N; g.ldk = bpl.ldk; g.E = 1; g.k = 1; g.Nout = int(I); g.K = int(H);
    TOPMOE_TRY(launch_gemm(KIND_BWD_GU, dtype, bpl.gu, g, (N + bpl.gu.bm - 1) / bpl.gu.bm, l0));
  } else if (N > 0) {
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
    dn.ksplit = pl.down_ksplit; dn.kchunk = pl.down_kchunk;
    dn.partial = reinterpret_cast<float*>(ws + pl.off_partial);
    TOPMOE_TRY(launch_down(dtype, pl.down, dn, (N + pl.down.bm - 1) / pl.down.bm, false, l1));
  }
  TOPMOE_TRY(st.close(l1));
  return TOPMOE_OK;
}

// The MoE forward; with `saved` (a backward workspace) as for the dense one.
int moe_fwd_impl(const void* x, const float* Wr, const void* Wg, const void* Wu, const void* Wd,
                 const void* residual, int64_t N, int64_t H, int64_t I, int E, int k,
                 float aux_coef, float z_coef, float capacity_factor, int flags, int dtype,
                 void* y, int32_t* topk_idx, float* alpha, float* aux_loss, float* z_loss,
                 int32_t* expert_offsets, int32_t* sorted_token_ids, void* workspace,
                 size_t workspace_bytes, void* saved, size_t saved_bytes, bool train,
                 void* stream, void* const* stage_events) {
  MoePlan pl;
  const int status = plan_moe(N, H, I, E, k, dtype, &pl);
  if (status != TOPMOE_OK) return status;
  MoeBwdPlan bpl;
  if (train) {
    const int bst = plan_moe_bwd(N, H, I, E, k, dtype, &bpl);
    if (bst != TOPMOE_OK) return bst;
    if (!saved) return TOPMOE_ERR_NULL_ARG;
    if (saved_bytes < bpl.total) return TOPMOE_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(saved, 256)) return TOPMOE_ERR_BAD_ARG;
  }
  // zero-size tensors (N == 0) are never touched and may be NULL
  if (!Wr || !Wg || !Wu || !Wd || !aux_loss || !workspace ||
      (N > 0 && (!x || !y || !topk_idx || !alpha)))
    return TOPMOE_ERR_NULL_ARG;
  if (!nonneg_finite(aux_coef) || !nonneg_finite(z_coef) || !nonneg_finite(capacity_factor))
    return TOPMOE_ERR_BAD_ARG;
  if (flags & ~(TOPMOE_MOE_RAW_TOPK_WEIGHTS | TOPMOE_MOE_EVAL)) return TOPMOE_ERR_BAD_ARG;
  const bool renorm = (flags & TOPMOE_MOE_RAW_TOPK_WEIGHTS) == 0;
  if (flags & TOPMOE_MOE_EVAL) {  // outside training the module adds no aux (or z) loss
    aux_coef = 0.f;
    z_coef = 0.f;
  }
  if (workspace_bytes < pl.total) return TOPMOE_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(Wg, 16) || !aligned(Wu, 16) ||
      !aligned(Wd, 16) || !aligned(residual, 16) || !aligned(y, 16) || !aligned(topk_idx, 4) ||
      !aligned(alpha, 4) || !aligned(aux_loss, 4) || !aligned(z_loss, 4) ||
      !aligned(expert_offsets, 4) || !aligned(sorted_token_ids, 4) || !aligned(workspace, 256))
    return TOPMOE_ERR_BAD_ARG;
  const int cap = capacity_of(capacity_factor, N, k, E);

  const Stages st{stage_events, static_cast<hipStream_t>(stream)};
  char* ws = static_cast<char*>(workspace);
  char* sv = static_cast<char*>(saved);
  // Training: the routing buffers are the backward workspace's own (the
  // backward keeps them at its start in this same layout), plus the
  // probabilities, logsumexps, selections and pre-capacity offsets the
  // backward needs, so that it takes the routing from there.
  char* rb = train ? sv : ws;
  int32_t* count_part = reinterpret_cast<int32_t*>(rb + pl.off_count_part);
  float* psum_part = reinterpret_cast<float*>(rb + pl.off_psum_part);
  int32_t* offsets = (expert_offsets && !train) ? expert_offsets
                                                : reinterpret_cast<int32_t*>(rb + pl.off_offsets);
  int32_t* sorted_entry = reinterpret_cast<int32_t*>(rb + pl.off_sorted);
  float* alpha_g = reinterpret_cast<float*>(rb + pl.off_alpha_g);
  float* z_part = reinterpret_cast<float*>(rb + pl.off_zpart);
  uint8_t* keep = cap > 0 ? reinterpret_cast<uint8_t*>(rb + pl.off_keep) : nullptr;
  int32_t* counts_off = train ? reinterpret_cast<int32_t*>(rb + pl.off_counts_off) : nullptr;
  float* probs = train ? reinterpret_cast<float*>(sv + bpl.off_probs) : nullptr;
  float* lse = train && z_coef != 0.f ? reinterpret_cast<float*>(sv + bpl.off_lse) : nullptr;
  int32_t* topk_keep = train ? reinterpret_cast<int32_t*>(sv + bpl.off_topk) : nullptr;
  float* alpha_keep = train ? reinterpret_cast<float*>(sv + bpl.off_alpha) : nullptr;
  int32_t* offsets_out = train ? expert_offsets : nullptr;  // the caller's copy
  void* h = ws + pl.off_h;
  void* slots = ws + pl.off_slots;

  if (N == 0) {
    for (int i = 0; i < TOPMOE_MOE_STAGES; ++i) {
      const Launch L = st.at(i);
      if (i == 1) {
        TOPMOE_TRY(launch_empty_route(E, offsets, aux_loss, z_loss, L));
        if (offsets_out) {
          Launch c = L;
          c.start = c.stop = nullptr;
          TOPMOE_TRY(launch_empty_route(E, offsets_out, aux_loss, z_loss, c));
        }
      }
      TOPMOE_TRY(st.close(L));
    }
    return TOPMOE_OK;
  }

  // Decode-sized inference calls take every token against every expert in
  // the gate/up projection (the weights stream the same; the MFMAs were idle)
  // and route in extra blocks of that same launch; the down projection then
  // groups the entries itself.
  const bool inline_route = !train && cap == 0 && pl.inline_ok;
  const bool allx = inline_route && pl.allx;
  // 0: router, softmax, top-k, alpha, per-block counts and sums of p
  const Launch l0 = st.at(0);
  if (!allx)
    TOPMOE_TRY(launch_router(x, Wr, dtype, N, int(H), E, k, renorm, pl.tb, pl.nblk,
                             pl.router_mode, topk_idx, alpha, probs, lse, count_part,
                             psum_part, z_part, l0));
  TOPMOE_TRY(st.close(l0));
  // 1: expert offsets, aux (and z) loss, stable scatter of entries into expert
  // groups (under a capacity: of the kept entries).  Decode-sized calls
  // (few entries, the 64 x 128 weight-streaming tiles) skip this launch: each
  // block of the two GEMMs groups the entries itself (GemmParams::inl_topk)
  // and one extra block of the gate/up launch (of the down launch when the
  // router runs inside the gate/up launch) writes these outputs.
  const Launch l1 = st.at(1);
  if (!inline_route)
    TOPMOE_TRY(launch_permute(count_part, psum_part, z_part, topk_idx, alpha, pl.nblk, E, k,
                              pl.tb, N, aux_coef, z_coef, cap, offsets, counts_off, aux_loss,
                              z_loss, sorted_entry, alpha_g, sorted_token_ids, keep, topk_keep,
                              alpha_keep, offsets_out, l1));
  TOPMOE_TRY(st.close(l1));
  auto set_inline = [&](GemmParams& g, bool outputs) {
    g.offsets = nullptr; g.entries = nullptr; g.alpha = nullptr;
    g.inl_topk = topk_idx; g.inl_alpha = alpha; g.inl_n = int(pl.rows); g.inl_nblk = pl.nblk;
    g.inl_tokens = N; g.inl_coef = aux_coef; g.inl_z_coef = z_coef;
    if (outputs) {
      g.inl_outputs = 1;
      g.inl_offsets_out = expert_offsets; g.inl_sorted_out = sorted_token_ids;
      g.inl_psum_part = psum_part; g.inl_z_part = z_part;
      g.inl_aux_out = aux_loss; g.inl_z_out = z_loss;
    }
  };
  // 2: grouped gate/up GEMM + SiLU * up (training: the backward's g, u
  // projection, keeping the pairs and h^T in `saved`, h row-major as well)
  const Launch l2 = st.at(2);
  if (train) {
    GemmParams g{};
    g.A = x; g.B0 = Wg; g.B1 = Wu; g.out = sv + bpl.off_gu; g.out1 = sv + bpl.off_hT;
    g.out2 = h;
    g.entries = sorted_entry; g.offsets = offsets;
    g.M = pl.rows; g.ldk = bpl.ldk; g.E = E; g.k = k; g.Nout = int(I); g.K = int(H);
    TOPMOE_TRY(launch_gemm(KIND_BWD_GU, dtype, bpl.gu, g, bpl.gu_mtiles, l2));
  } else {
    GemmParams up{};
    up.A = x; up.B0 = Wg; up.B1 = Wu; up.out = h;
    up.entries = sorted_entry; up.offsets = offsets; up.alpha = nullptr;
    up.M = pl.rows; up.E = E; up.k = k; up.Nout = int(I); up.K = int(H);
    int64_t up_mtiles = pl.up_mtiles;
    if (allx) {
      up.entries = nullptr; up.offsets = nullptr;
      up.allx_n = N;
      up_mtiles = int64_t(E) * ((N + pl.up.bm - 1) / pl.up.bm);
      up.rt_wr = Wr; up.rt_blocks = pl.nblk; up.rt_tb = pl.tb; up.rt_renorm = renorm ? 1 : 0;
      up.rt_n = N; up.rt_topk = topk_idx; up.rt_alpha = alpha;
      up.rt_count = count_part; up.rt_psum = psum_part; up.rt_zpart = z_part;
    } else if (inline_route) {
      set_inline(up, true);
    }
    TOPMOE_TRY(launch_gemm(KIND_GATEUP, dtype, pl.up, up, up_mtiles, l2));
  }
  TOPMOE_TRY(st.close(l2));
  // 3: grouped down GEMM, alpha-scaled, into y (k == 1) or the slots
  const bool direct = k == 1;
  const Launch l3 = st.at(3);
  GemmParams dn{};
  dn.A = h; dn.B0 = Wd; dn.B1 = nullptr; dn.out = direct ? y : slots;
  dn.residual = direct ? residual : nullptr;  // otherwise added by the combine
  dn.entries = sorted_entry; dn.offsets = offsets; dn.alpha = alpha_g;
  dn.M = pl.rows; dn.E = E; dn.k = k; dn.Nout = int(H); dn.K = int(I);
  dn.ksplit = pl.down_ksplit; dn.kchunk = pl.down_kchunk;
  dn.partial = reinterpret_cast<float*>(ws + pl.off_partial);
  if (inline_route) set_inline(dn, allx);  // with every token against every expert, the
  if (allx) dn.allx_n = N;                  // down launch writes the routing outputs
  TOPMOE_TRY(launch_down(dtype, pl.down, dn, pl.down_mtiles, !direct, l3));
  TOPMOE_TRY(st.close(l3));
  // 4: fixed-order combine of the kept slots (k == 1 under a capacity: the
  // dropped tokens' rows of y, which the down GEMM did not write)
  const Launch l4 = st.at(4);
  if (!direct)
    TOPMOE_TRY(launch_combine(slots, topk_idx, keep, residual, N, int(H), k, dtype, y, l4));
  else if (cap > 0)
    TOPMOE_TRY(launch_combine(nullptr, topk_idx, keep, residual, N, int(H), k, dtype, y, l4));
  TOPMOE_TRY(st.close(l4));
  return TOPMOE_OK;
}

}  // namespace

extern "C" {

int ffn_swiglu_fwd(const void* x, const void* Wg, const void* Wu, const void* Wd,
                   const void* residual, void* y, int64_t N, int64_t H, int64_t I, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream,
                   void* const* stage_events) {
  return ffn_fwd_impl(x, Wg, Wu, Wd, residual, y, N, H, I, dtype, workspace, workspace_bytes,
                      nullptr, 0, false, stream, stage_events);
}

int ffn_swiglu_fwd_train(const void* x, const void* Wg, const void* Wu, const void* Wd,
                         const void* residual, void* y, int64_t N, int64_t H, int64_t I,
                         int dtype, void* workspace, size_t workspace_bytes, void* saved,
                         size_t saved_bytes, void* stream, void* const* stage_events) {
  return ffn_fwd_impl(x, Wg, Wu, Wd, residual, y, N, H, I, dtype, workspace, workspace_bytes,
                      saved, saved_bytes, true, stream, stage_events);
}

int moe_ffn_fwd(const void* x, const float* Wr, const void* Wg, const void* Wu, const void* Wd,
                const void* residual, int64_t N, int64_t H, int64_t I, int E, int k,
                float aux_coef, float z_coef, float capacity_factor, int flags, int dtype,
                void* y, int32_t* topk_idx, float* alpha, float* aux_loss, float* z_loss,
                int32_t* expert_offsets, int32_t* sorted_token_ids, void* workspace,
                size_t workspace_bytes, void* stream, void* const* stage_events) {
  return moe_fwd_impl(x, Wr, Wg, Wu, Wd, residual, N, H, I, E, k, aux_coef, z_coef,
                      capacity_factor, flags, dtype, y, topk_idx, alpha, aux_loss, z_loss,
                      expert_offsets, sorted_token_ids, workspace, workspace_bytes, nullptr, 0,
                      false, stream, stage_events);
}

int moe_ffn_fwd_train(const void* x, const float* Wr, const void* Wg, const void* Wu,
                      const void* Wd, const void* residual, int64_t N, int64_t H, int64_t I,
                      int E, int k, float aux_coef, float z_coef, float capacity_factor,
                      int flags, int dtype, void* y, int32_t* topk_idx, float* alpha,
                      float* aux_loss, float* z_loss, int32_t* expert_offsets,
                      int32_t* sorted_token_ids, void* workspace, size_t workspace_bytes,
                      void* saved, size_t saved_bytes, void* stream, void* const* stage_events) {
  return moe_fwd_impl(x, Wr, Wg, Wu, Wd, residual, N, H, I, E, k, aux_coef, z_coef,
                      capacity_factor, flags, dtype, y, topk_idx, alpha, aux_loss, z_loss,
                      expert_offsets, sorted_token_ids, workspace, workspace_bytes, saved,
                      saved_bytes, true, stream, stage_events);
}

}  // extern "C"

// The workspace of moe_ffn_fwd_noalloc, for callers that cannot allocate:
// a fixed array in device memory that every GPU the library runs on holds
// until the process ends.  In host code `scratch` is only a stand-in for the
// array; its device address comes from hipGetSymbolAddress.
constexpr size_t kNoallocScratchBytes = TOPMOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};  // device address of `scratch`, per device

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return TOPMOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return TOPMOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TOPMOE_OK;
}

}  // namespace

extern "C" {

int moe_ffn_fwd_noalloc(const void* x, const float* Wr, const void* Wg, const void* Wu,
                        const void* Wd, const void* residual, int64_t N, int64_t H, int64_t I,
                        int E, int k, float aux_coef, float z_coef, float capacity_factor,
                        int flags, int dtype, void* y, int32_t* topk_idx, float* alpha,
                        float* aux_loss, float* z_loss, int32_t* expert_offsets,
                        int32_t* sorted_token_ids, void* stream, void* const* stage_events) {
  MoePlan pl;
  const int status = plan_moe(N, H, I, E, k, dtype, &pl);
  if (status != TOPMOE_OK) return status;
  if (pl.total > kNoallocScratchBytes) return TOPMOE_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  const int st = scratch_on_current_device(&ws);
  if (st != TOPMOE_OK) return st;
  // every buffer the forward reads from its workspace it first writes in the
  // same call, so nothing there needs clearing between calls
  return moe_fwd_impl(x, Wr, Wg, Wu, Wd, residual, N, H, I, E, k, aux_coef, z_coef,
                      capacity_factor, flags, dtype, y, topk_idx, alpha, aux_loss, z_loss,
                      expert_offsets, sorted_token_ids, ws, kNoallocScratchBytes, nullptr, 0,
                      false, stream, stage_events);
}

size_t ffn_bwd_workspace_bytes(int64_t N, int64_t H, int64_t I, int dtype) {
  FfnBwdPlan pl;
  return plan_ffn_bwd(N, H, I, dtype, &pl) == TOPMOE_OK ? pl.total : 0;
}

size_t moe_bwd_workspace_bytes(int64_t N, int64_t H, int64_t I, int E, int k, int dtype) {
  MoeBwdPlan pl;
  return plan_moe_bwd(N, H, I, E, k, dtype, &pl) == TOPMOE_OK ? pl.total : 0;
}

}  // extern "C"

namespace {

// The dense backward; `saved`: the workspace already holds the pairs (g, u)
// and h^T from ffn_swiglu_fwd_train on the same inputs (stage 2 is skipped).
int ffn_bwd_impl(const void* x, const void* Wg, const void* Wu, const void* Wd, const void* dy,
                 void* dx, void* dWg, void* dWu, void* dWd, int64_t N, int64_t H, int64_t I,
                 int dtype, void* workspace, size_t workspace_bytes, bool saved, void* stream,
                 void* const* stage_events) {
  FfnBwdPlan pl;
  const int status = plan_ffn_bwd(N, H, I, dtype, &pl);
  if (status != TOPMOE_OK) return status;
  if (!Wg || !Wu || !Wd || !dWg || !dWu || !dWd || !workspace || (N > 0 && (!x || !dy || !dx)))
    return TOPMOE_ERR_NULL_ARG;
  if (workspace_bytes < pl.total) return TOPMOE_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(x, 16) || !aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) ||
      !aligned(dy, 16) || !aligned(dx, 16) || !aligned(dWg, 16) || !aligned(dWu, 16) ||
      !aligned(dWd, 16) || !aligned(workspace, 256))
    return TOPMOE_ERR_BAD_ARG;

  const Stages st{stage_events, static_cast<hipStream_t>(stream)};
  char* ws = static_cast<char*>(workspace);
  void* wgT = ws + pl.off_wgT;
  void* wdT = ws + pl.off_wdT;
  void* xT = ws + pl.off_xT;
  void* dyT = ws + pl.off_dyT;
  void* gu = ws + pl.off_gu;
  void* dgdu = ws + pl.off_dgdu;
  void* dgT = ws + pl.off_dgT;
  void* duT = ws + pl.off_duT;
  void* hT = ws + pl.off_hT;
  const int iH = int(H), iI = int(I);

  // 0: weight transposes: [Wg | Wu]^T [H, 2I] and Wd^T [I, H]
  const Launch l0 = st.at(0);
  {
    TransposeJobs tj{};
    tj.job[0] = TransposeJob{Wg, wgT, iI, iH, 1, 0, 2 * I, 0, 0};
    tj.job[1] = TransposeJob{Wu, wgT, iI, iH, 1, iI, 2 * I, 0, 0};
    tj.job[2] = TransposeJob{Wd, wdT, iH, iI, 1, 0, H, 0, 0};
    tj.n = 3;
    TOPMOE_TRY(launch_transpose(dtype, tj, int((I / 64) * (H / 64)), 1, l0));
  }
  TOPMOE_TRY(st.close(l0));
  // 1: activation transposes x^T, dy^T [H, ldk] (zero columns past N)
  const Launch l1 = st.at(1);
  {
    GatherTransposeJobs gj{};
    gj.job[0] = GatherTransposeJob{x, xT, nullptr};
    gj.job[1] = GatherTransposeJob{dy, dyT, nullptr};
    gj.n = 2;
    gj.offsets = nullptr; gj.entries = nullptr;
    gj.E = 1; gj.k = 1; gj.C = iH; gj.rows = N; gj.ldo = pl.ldk;
    TOPMOE_TRY(launch_gather_transpose(dtype, gj, pl.ldk, l1));
  }
  TOPMOE_TRY(st.close(l1));
  // 2: g, u recomputed: the pairs (g, u) and h^T (kept by the training forward)
  const Launch l2 = st.at(2);
  if (N > 0 && !saved) {
    GemmParams g{};
    g.A = x; g.B0 = Wg; g.B1 = Wu; g.out = gu; g.out1 = hT;
    g.M = N; g.ldk = pl.ldk; g.E = 1; g.k = 1; g.Nout = iI; g.K = iH;
    TOPMOE_TRY(launch_gemm(KIND_BWD_GU, dtype, pl.gu, g, (N + pl.gu.bm - 1) / pl.gu.bm, l2));
  }
  TOPMOE_TRY(st.close(l2));
  // 3: dh = dy Wd, then [dg | du], dg^T, du^T
  const Launch l3 = st.at(3);
  if (N > 0) {
    GemmParams g{};
    g.A = dy; g.B0 = wdT; g.gu = gu; g.out = dgdu; g.out1 = dgT; g.out2 = duT;
    g.M = N; g.ldk = pl.ldk; g.E = 1; g.k = 1; g.Nout = iI; g.K = iH;
    TOPMOE_TRY(launch_gemm(KIND_BWD_DH, dtype, pl.dh, g, (N + pl.dh.bm - 1) / pl.dh.bm, l3));
  }
  TOPMOE_TRY(st.close(l3));
  // 4: dx = [dg | du] [Wg | Wu]
  const Launch l4 = st.at(4);
  if (N > 0) {
    GemmParams g{};
    g.A = dgdu; g.B0 = wgT; g.out = dx;
    g.M = N; g.E = 1; g.k = 1; g.Nout = iH; g.K = 2 * iI;
    TOPMOE_TRY(launch_gemm(KIND_DOWN_Y, dtype, pl.dx, g, (N + pl.dx.bm - 1) / pl.dx.bm, l4));
  }
  TOPMOE_TRY(st.close(l4));
  // 5: dWg = dg^T x, dWu = du^T x (contraction over tokens)
  const Launch l5 = st.at(5);
  {
    GemmParams g{};
    g.A = dgT; g.A1 = duT; g.B0 = xT; g.out = dWg; g.out1 = dWu;
    g.M = I; g.ldk = pl.ldk; g.kcount = N; g.E = 1; g.k = 1; g.Nout = iH; g.K = int(pl.ldk);
    TOPMOE_TRY(launch_gemm(KIND_WGRAD2, dtype, pl.wgu, g, 0, l5));
  }
  TOPMOE_TRY(st.close(l5));
  // 6: dWd = dy^T h
  const Launch l6 = st.at(6);
  {
    GemmParams g{};
    g.A = dyT; g.B0 = hT; g.out = dWd;
    g.M = H; g.ldk = pl.ldk; g.kcount = N; g.E = 1; g.k = 1; g.Nout = iI; g.K = int(pl.ldk);
    TOPMOE_TRY(launch_gemm(KIND_WGRAD1, dtype, pl.wd, g, 0, l6));
  }
  TOPMOE_TRY(st.close(l6));
  return TOPMOE_OK;
}

}  // namespace

extern "C" {

int ffn_swiglu_bwd(const void* x, const void* Wg, const void* Wu, const void* Wd, const void* dy,
                   void* dx, void* dWg, void* dWu, void* dWd, int64_t N, int64_t H, int64_t I,
                   int dtype, void* workspace, size_t workspace_bytes, void* stream,
                   void* const* stage_events) {
  return ffn_bwd_impl(x, Wg, Wu, Wd, dy, dx, dWg, dWu, dWd, N, H, I, dtype, workspace,
                      workspace_bytes, false, stream, stage_events);
}

int ffn_swiglu_bwd_saved(const void* x, const void* Wg, const void* Wu, const void* Wd,
                         const void* dy, void* dx, void* dWg, void* dWu, void* dWd, int64_t N,
                         int64_t H, int64_t I, int dtype, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* stage_events) {
  return ffn_bwd_impl(x, Wg, Wu, Wd, dy, dx, dWg, dWu, dWd, N, H, I, dtype, workspace,
                      workspace_bytes, true, stream, stage_events);
}

int moe_ffn_bwd(const void* x, const float* Wr, const void* Wg, const void* Wu, const void* Wd,
                const void* dy, float aux_grad, float z_grad, const float* aux_grad_scale,
                const float* z_grad_scale, int64_t N, int64_t H, int64_t I,
                int E, int k, float aux_coef, float z_coef, float capacity_factor, int flags,
                int dtype, void* dx, float* dWr, void* dWg, void* dWu, void* dWd, void* workspace,
                size_t workspace_bytes, void* stream, void* const* stage_events) {
  MoeBwdPlan pl;
  const int status = plan_moe_bwd(N, H, I, E, k, dtype, &pl);
  if (status != TOPMOE_OK) return status;
  if (!Wr || !Wg || !Wu || !Wd || !dWr || !dWg || !dWu || !dWd || !workspace ||
      (N > 0 && (!x || !dy || !dx)))
    return TOPMOE_ERR_NULL_ARG;
  if (!nonneg_finite(aux_coef) || !nonneg_finite(z_coef) || !nonneg_finite(capacity_factor) ||
      !isfinite(aux_grad) || !isfinite(z_grad))
    return TOPMOE_ERR_BAD_ARG;
  if (flags & ~(TOPMOE_MOE_RAW_TOPK_WEIGHTS | TOPMOE_MOE_BWD_SAVED | TOPMOE_MOE_EVAL))
    return TOPMOE_ERR_BAD_ARG;
  if (!aligned(aux_grad_scale, 4) || !aligned(z_grad_scale, 4)) return TOPMOE_ERR_BAD_ARG;
  if (flags & TOPMOE_MOE_EVAL) {  // outside training: no aux or z-loss term
    aux_coef = 0.f;
    z_coef = 0.f;
  }
  const int cap = capacity_of(capacity_factor, N, k, E);
  const bool renorm = (flags & TOPMOE_MOE_RAW_TOPK_WEIGHTS) == 0;
  const bool saved = (flags & TOPMOE_MOE_BWD_SAVED) != 0;
  if (workspace_bytes < pl.total) return TOPMOE_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(Wg, 16) || !aligned(Wu, 16) ||
      !aligned(Wd, 16) || !aligned(dy, 16) || !aligned(dx, 16) || !aligned(dWr, 16) ||
      !aligned(dWg, 16) || !aligned(dWu, 16) || !aligned(dWd, 16) || !aligned(workspace, 256))
    return TOPMOE_ERR_BAD_ARG;

  const MoePlan& rp = pl.route;
  const Stages st{stage_events, static_cast<hipStream_t>(stream)};
  char* ws = static_cast<char*>(workspace);
  int32_t* count_part = reinterpret_cast<int32_t*>(ws + rp.off_count_part);
  float* psum_part = reinterpret_cast<float*>(ws + rp.off_psum_part);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + rp.off_offsets);
  int32_t* sorted_entry = reinterpret_cast<int32_t*>(ws + rp.off_sorted);
  float* alpha_g = reinterpret_cast<float*>(ws + rp.off_alpha_g);
  float* probs = reinterpret_cast<float*>(ws + pl.off_probs);
  float* lse = reinterpret_cast<float*>(ws + pl.off_lse);
  float* z_part = reinterpret_cast<float*>(ws + rp.off_zpart);
  int32_t* counts_off = reinterpret_cast<int32_t*>(ws + rp.off_counts_off);
  uint8_t* keep = cap > 0 ? reinterpret_cast<uint8_t*>(ws + rp.off_keep) : nullptr;
  int32_t* topk_idx = reinterpret_cast<int32_t*>(ws + pl.off_topk);
  float* alpha = reinterpret_cast<float*>(ws + pl.off_alpha);
  float* aux = reinterpret_cast<float*>(ws + pl.off_aux);
  void* wgT = ws + pl.off_wgT;
  void* wdT = ws + pl.off_wdT;
  void* xT = ws + pl.off_xT;
  void* dyT = ws + pl.off_dyT;
  void* gu = ws + pl.off_gu;
  void* dgdu = ws + pl.off_dgdu;
  void* dgT = ws + pl.off_dgT;
  void* duT = ws + pl.off_duT;
  void* hT = ws + pl.off_hT;
  float* dal = reinterpret_cast<float*>(ws + pl.off_dal);
  void* slots = ws + pl.off_slots;
  float* dr = reinterpret_cast<float*>(ws + pl.off_dr);
  float* dwr_part = reinterpret_cast<float*>(ws + pl.off_dwr);
  const int iH = int(H), iI = int(I);
  const int64_t rows = rp.rows;

  // 0, 1: the forward's routing (probabilities kept for the softmax backward);
  // with a saved workspace the training forward left it there
  const Launch l0 = st.at(0);
  if (N > 0 && !saved)
    TOPMOE_TRY(launch_router(x, Wr, dtype, N, iH, E, k, renorm, rp.tb, rp.nblk, rp.router_mode,
                             topk_idx, alpha, probs, z_coef != 0.f ? lse : nullptr, count_part,
                             psum_part, z_part, l0));
  TOPMOE_TRY(st.close(l0));
  const Launch l1 = st.at(1);
  if (N > 0 && !saved)
    TOPMOE_TRY(launch_permute(count_part, psum_part, z_part, topk_idx, alpha, rp.nblk, E, k,
                              rp.tb, N, aux_coef, z_coef, cap, offsets, counts_off, aux, nullptr,
                              sorted_entry, alpha_g, nullptr, keep, nullptr, nullptr, nullptr,
                              l1));
  else if (!saved)
    TOPMOE_TRY(launch_empty_route(E, offsets, aux, nullptr, l1));
  TOPMOE_TRY(st.close(l1));
  // 2: per-expert weight transposes: [Wg | Wu]^T [E, H, 2I], Wd^T [E, I, H]
  const Launch l2 = st.at(2);
  {
    TransposeJobs tj{};
    const int64_t ih = I * H;
    tj.job[0] = TransposeJob{Wg, wgT, iI, iH, E, 0, 2 * I, ih, 2 * ih};
    tj.job[1] = TransposeJob{Wu, wgT, iI, iH, E, iI, 2 * I, ih, 2 * ih};
    tj.job[2] = TransposeJob{Wd, wdT, iH, iI, E, 0, H, ih, ih};
    tj.n = 3;
    TOPMOE_TRY(launch_transpose(dtype, tj, int((I / 64) * (H / 64)), E, l2));
  }
  TOPMOE_TRY(st.close(l2));
  // 3: x^T and (alpha dy)^T in expert-grouped padded columns
  const Launch l3 = st.at(3);
  {
    GatherTransposeJobs gj{};
    gj.job[0] = GatherTransposeJob{x, xT, nullptr};
    gj.job[1] = GatherTransposeJob{dy, dyT, alpha_g};
    gj.n = N > 0 ? 2 : 0;
    gj.offsets = offsets; gj.entries = sorted_entry;
    gj.E = E; gj.k = k; gj.C = iH; gj.rows = rows; gj.ldo = pl.ldk;
    TOPMOE_TRY(launch_gather_transpose(dtype, gj, pl.ldk, l3));
  }
  TOPMOE_TRY(st.close(l3));
  // 4: per expert g, u recomputed: the pairs (g, u) and h^T (kept by the
  // training forward)
  const Launch l4 = st.at(4);
  if (N > 0 && !saved) {
    GemmParams g{};
    g.A = x; g.B0 = Wg; g.B1 = Wu; g.out = gu; g.out1 = hT;
    g.entries = sorted_entry; g.offsets = offsets;
    g.M = rows; g.ldk = pl.ldk; g.E = E; g.k = k; g.Nout = iI; g.K = iH;
    TOPMOE_TRY(launch_gemm(KIND_BWD_GU, dtype, pl.gu, g, pl.gu_mtiles, l4));
  }
  TOPMOE_TRY(st.close(l4));
  // 5: per expert dh = alpha dy Wd: [dg | du], dg^T, du^T, d alpha partials
  const Launch l5 = st.at(5);
  if (N > 0) {
    GemmParams g{};
    g.A = dy; g.B0 = wdT; g.gu = gu;
    g.out = dgdu; g.out1 = dgT; g.out2 = duT; g.dalpha_part = dal;
    g.entries = sorted_entry; g.offsets = offsets; g.alpha = alpha_g;
    g.M = rows; g.ldk = pl.ldk; g.E = E; g.k = k; g.Nout = iI; g.K = iH;
    TOPMOE_TRY(launch_gemm(KIND_BWD_DH, dtype, pl.dh, g, pl.dh_mtiles, l5));
  }
  TOPMOE_TRY(st.close(l5));
  // 6: per entry dx term [dg | du] [Wg_e | Wu_e] into its slot
  const Launch l6 = st.at(6);
  if (N > 0) {
    GemmParams g{};
    g.A = dgdu; g.B0 = wgT; g.out = slots;
    g.entries = sorted_entry; g.offsets = offsets; g.alpha = nullptr;
    g.M = rows; g.E = E; g.k = k; g.Nout = iH; g.K = 2 * iI;
    TOPMOE_TRY(launch_gemm(KIND_DOWN_SLOTS, dtype, pl.dx, g, pl.dx_mtiles, l6));
  }
  TOPMOE_TRY(st.close(l6));
  // 7: router backward: d alpha -> dp (renormalisation, aux) -> softmax -> dr
  const Launch l7 = st.at(7);
  {
    const double scale = N > 0 ? double(aux_grad) * double(aux_coef) * double(E) /
                                     (double(N) * double(N))
                               : 0.0;
    const double zscale = N > 0 ? double(z_grad) * double(z_coef) * 2.0 / double(N) : 0.0;
    TOPMOE_TRY(launch_router_bwd(probs, topk_idx, dal, pl.nt_h, counts_off, keep,
                                 z_coef != 0.f ? lse : nullptr, N, E, k, renorm, float(scale),
                                 aux_grad_scale, float(zscale), z_grad_scale, dr, l7));
  }
  TOPMOE_TRY(st.close(l7));
  // 8: dx = sum of the slots (ascending expert) + W_r^T dr
  const Launch l8 = st.at(8);
  TOPMOE_TRY(launch_combine_bwd(slots, topk_idx, keep, dr, Wr, N, iH, E, k, dtype, dx, l8));
  TOPMOE_TRY(st.close(l8));
  // 9: dW_r = dr^T x
  const Launch l9 = st.at(9);
  TOPMOE_TRY(launch_dwr(x, dr, N, iH, E, dtype, dwr_part, dWr, l9));
  TOPMOE_TRY(st.close(l9));
  // 10: dWg_e = dg_e^T x_e, dWu_e = du_e^T x_e over each expert's rows
  const Launch l10 = st.at(10);
  {
    GemmParams g{};
    g.A = dgT; g.A1 = duT; g.B0 = xT; g.out = dWg; g.out1 = dWu;
    g.offsets = offsets;
    g.M = I; g.ldk = pl.ldk; g.E = E; g.k = k; g.Nout = iH; g.K = int(pl.ldk);
    TOPMOE_TRY(launch_gemm(KIND_WGRAD2, dtype, pl.wgu, g, 0, l10));
  }
  TOPMOE_TRY(st.close(l10));
  // 11: dWd_e = (alpha dy)_e^T h_e
  const Launch l11 = st.at(11);
  {
    GemmParams g{};
    g.A = dyT; g.B0 = hT; g.out = dWd;
    g.offsets = offsets;
    g.M = H; g.ldk = pl.ldk; g.E = E; g.k = k; g.Nout = iI; g.K = int(pl.ldk);
    TOPMOE_TRY(launch_gemm(KIND_WGRAD1, dtype, pl.wd, g, 0, l11));
  }
  TOPMOE_TRY(st.close(l11));
  return TOPMOE_OK;
}

int topmoe_set_tile_override(int gemm, const int* shape) { return set_tile_override(gemm, shape); }

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
