// Host-side planning for the FFN / MoE forward: argument validation, the
// workspace layout and launch-shape choices.  Plain C++ (no HIP types) so the
// same logic is testable on a machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace topmoe {

enum GemmKind {
  KIND_GATEUP = 0,      // h = SiLU(A Wg^T) * (A Wu^T), rows gathered from x
  KIND_DOWN_Y = 1,      // y[token] = alpha * (h Wd^T), written in the output dtype
  KIND_DOWN_SLOTS = 2,  // slot[entry] = alpha * (h Wd^T), in the operand dtype
  // backward
  KIND_BWD_GU = 3,      // g, u = x Wg^T, x Wu^T (rows gathered from x): writes the pairs
                        // (g, u) row-major and h^T in padded group columns
  KIND_WGRAD2 = 4,      // out0 = A0 B^T, out1 = A1 B^T per group, K = the group's padded rows
  KIND_WGRAD1 = 5,      // out0 = A0 B^T per group, K = the group's padded rows
  KIND_DOWN_PARTIAL = 7,  // the down projection split along K: each work item (a tile and a
                          // K chunk) writes its raw fp32 sums to GemmParams::partial
  KIND_BWD_DH = 6,      // dh = alpha * dy Wd (rows gathered from dy), with the pairs (g, u):
                        // writes [dg | du] row-major, dg^T / du^T in padded group columns and
                        // per-row partial sums of dh_raw . h (d alpha)
};

constexpr size_t kAlign = 256;
constexpr int kDwrChunk = 64;   // tokens per partial of the router-weight gradient

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

// One GEMM launch shape: block tile BM x BN (per output matrix) and the
// depth of the LDS ring of K slices.
struct GemmShape {
  int bm = 0, bn = 0;      // block tile
  int wm = 2, wn = 2;      // wavefront grid (wm * wn wavefronts of 64 lanes)
  int rb = 128;            // LDS row bytes per K slice
  int stages = 2;          // ring depth
};

struct FfnPlan {
  int64_t N = 0, H = 0, I = 0;
  int dtype = 0;
  int elem = 0;            // bytes per x / W / y element
  GemmShape up, down;      // gate/up and down GEMM tiles
  int down_ksplit = 1;     // K chunks of the down GEMM (1: not split)
  int down_kchunk = 0;     // K slices per chunk
  size_t off_h = 0;        // SiLU(g)*u intermediate [N, I]
  size_t off_partial = 0;  // f32 [down_ksplit, N, H] split-K partial sums (when split)
  size_t total = 0;        // workspace bytes
};

// Most K chunks of a split down projection.
constexpr int kMaxDownSplit = 6;

// Most entries (N * k) the in-block routing of a GEMM takes.
constexpr int kInlineMaxEntries = 512;

struct MoePlan {
  int64_t N = 0, H = 0, I = 0;
  int E = 0, k = 0, dtype = 0;
  int elem = 0;
  int64_t rows = 0;        // N * k expert rows
  int tb = 0;              // router / scatter tokens per block
  int nblk = 0;            // router / scatter blocks
  int router_mode = 0;     // 0 / 2: W_router in LDS, 4 / 16 lanes per token; 1: H split per token
  GemmShape up, down;
  int64_t up_mtiles = 0;   // upper bound on grouped M tiles (gate/up)
  int64_t down_mtiles = 0; // upper bound on grouped M tiles (down)
  // workspace layout (byte offsets)
  size_t off_count_part = 0;  // int32 [E, nblk] per-block expert counts
  size_t off_psum_part = 0;   // f32   [E, nblk] per-block sums of p
  size_t off_offsets = 0;     // int32 [E+1] expert offsets (when the caller passes none)
  size_t off_counts_off = 0;  // int32 [E+1] offsets of every selection (before a capacity)
  size_t off_zpart = 0;       // f32   [nblk] per-block sums of logsumexp^2 (z-loss)
  size_t off_keep = 0;        // u8    [N*k] 1 where an entry survives the capacity
  size_t off_sorted = 0;      // int32 [N*k] entry ids (t*k + j) grouped by expert
  size_t off_alpha_g = 0;     // f32   [N*k] alpha of each grouped row
  size_t off_h = 0;           // elem  [N*k, I] SiLU(g)*u in grouped row order
  size_t off_slots = 0;       // elem  [N*k, H] alpha-scaled expert outputs (k >= 2)
  int down_ksplit = 1;        // K chunks of the down GEMM (1: not split)
  int down_kchunk = 0;        // K slices per chunk
  size_t off_partial = 0;     // f32   [down_ksplit, N*k, H] split-K partial sums
  // few entries (at most kInlineMaxEntries), both projections on the 64 x 128
  // weight-streaming tile, the down projection unsplit: inference calls
  // without a capacity group the entries inside the GEMMs (in-block routing)
  bool inline_ok = false;
  // and with the split router at one token per block, E <= 16 and at most
  // one row tile of tokens, the gate/up projection can take every token
  // against every expert (h then holds E * N rows, group e's row t at
  // e * N + t), with the router's blocks in the same launch
  bool allx = false;
  size_t total = 0;
};

// Backward of the dense FFN.  Transposed activations keep tokens along
// their rows, padded to ldk = round64(N) columns (zeros past N), so the
// weight gradients contract over whole 64-token slices.
struct FfnBwdPlan {
  int64_t N = 0, H = 0, I = 0;
  int dtype = 0, elem = 0;
  int64_t ldk = 0;
  GemmShape gu, dh, dx, wgu, wd;  // g/u, dh, dx, dWg+dWu, dWd GEMMs
  size_t off_wgT = 0;    // [H, 2I]  [Wg | Wu]^T
  size_t off_wdT = 0;    // [I, H]   Wd^T
  size_t off_xT = 0;     // [H, ldk] x^T
  size_t off_dyT = 0;    // [H, ldk] dy^T
  size_t off_gu = 0;     // [N, I]   pairs (g, u)
  size_t off_dgdu = 0;   // [N, 2I]  [dg | du]
  size_t off_dgT = 0;    // [I, ldk] dg^T
  size_t off_duT = 0;    // [I, ldk] du^T
  size_t off_hT = 0;     // [I, ldk] h^T
  size_t total = 0;
};

// Backward of the MoE FFN: the forward's routing is recomputed (same kernels,
// so the same choices), then the expert GEMMs run on expert-grouped rows.
// Transposed activations hold each expert's rows in columns padded to a
// multiple of 64 (zeros in between); ldk bounds their total width.
struct MoeBwdPlan {
  MoePlan route;          // router / permutation parameters and buffers
  int64_t ldk = 0;
  GemmShape gu, dh, dx, wgu, wd;
  int64_t gu_mtiles = 0, dh_mtiles = 0, dx_mtiles = 0;
  int nt_h = 0;           // column tiles of the dh GEMM: d alpha partials per entry
  int nchunk = 0;         // token chunks of the router-weight gradient
  size_t off_probs = 0;   // f32 [N, E] softmax
  size_t off_lse = 0;     // f32 [N] logsumexp of the logits (z-loss backward)
  size_t off_topk = 0;    // i32 [N, k]
  size_t off_alpha = 0;   // f32 [N, k]
  size_t off_aux = 0;     // f32 [1] (forward value, unused)
  size_t off_wgT = 0;     // [E, H, 2I]
  size_t off_wdT = 0;     // [E, I, H]
  size_t off_xT = 0;      // [H, ldk]
  size_t off_dyT = 0;     // [H, ldk] (alpha * dy)^T
  size_t off_gu = 0;      // [N*k, I] pairs (g, u)
  size_t off_dgdu = 0;    // [N*k, 2I]
  size_t off_dgT = 0;     // [I, ldk]
  size_t off_duT = 0;     // [I, ldk]
  size_t off_hT = 0;      // [I, ldk]
  size_t off_dal = 0;     // f32 [N*k, nt_h]
  size_t off_slots = 0;   // [N*k, H] per-entry dx terms
  size_t off_dr = 0;      // f32 [N, E] router-logit gradients
  size_t off_dwr = 0;     // f32 [nchunk, E, H] partial router-weight gradients
  size_t total = 0;
};

// Returns TOPMOE_OK or a negative status; fills `plan` on success.
int plan_ffn(int64_t N, int64_t H, int64_t I, int dtype, FfnPlan* plan);
int plan_moe(int64_t N, int64_t H, int64_t I, int E, int k, int dtype, MoePlan* plan);
int plan_ffn_bwd(int64_t N, int64_t H, int64_t I, int dtype, FfnBwdPlan* plan);
int plan_moe_bwd(int64_t N, int64_t H, int64_t I, int E, int k, int dtype, MoeBwdPlan* plan);

// Launch shape for an M x Nout x K GEMM with `groups` row groups (experts).
GemmShape choose_gateup_tile(int64_t M, int64_t Nout, int64_t K, int groups, int dtype);
GemmShape choose_down_tile(int64_t M, int64_t Nout, int64_t K, int groups, int dtype);

// Whether the GEMM kernels of `kind` (a GemmKind) are instantiated with
// launch shape `sh` for `dtype` (defined beside the kernels; host code).
bool gemm_shape_supported(int kind, int dtype, const GemmShape& sh);

// Launch-shape overrides, for tuning sweeps and tests: one per GEMM of the
// path (the TOPMOE_TILE_* slots of include/topmoe.h).  Initialised once from
// the environment (TOPMOE_GATEUP_TILE, TOPMOE_DOWN_TILE, TOPMOE_BWDGU_TILE,
// TOPMOE_BWDDH_TILE, TOPMOE_WGU_TILE, TOPMOE_WD_TILE: "BMxBNxWMxWNxRBxS"),
// then set through set_tile_override.
int set_tile_override(int slot, const int* shape);

// K split of a down projection of `tiles` output tiles over K: chunks of
// *kchunk slices (RB bytes of each row), *ksplit of them, each non-empty;
// *ksplit = 1 when the tiles alone occupy at least half the CUs.
void choose_down_split(int64_t tiles, int64_t K, int elem, const GemmShape& sh, int* ksplit,
                       int* kchunk);

// Upper bound on the number of BM-row tiles over `groups` groups of total M rows.
inline int64_t grouped_mtiles_bound(int64_t M, int groups, int bm) {
  if (M <= 0) return 0;
  int64_t g = groups < M ? groups : M;
  return (M + bm - 1) / bm + (groups > 1 ? g : 0);
}

}  // namespace topmoe
