// Host-side planning: validation, workspace layout, launch shapes.
#include "plan.h"

#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "../../include/topmoe.h"

namespace topmoe {

namespace {

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;  // int32 row / entry ids
// The GEMMs address operand rows with 32-bit byte offsets from a per-matrix
// (per-expert for weights) base, so each operand matrix stays below 4 GiB.
// (Products are formed in double: exact below 2^53, and anything near or past
// that is far over the limit anyway.)
bool operand_ok(int64_t rows, int64_t cols, int elem) {
  return double(rows) * double(cols) * double(elem) < 4294967296.0;
}

bool dtype_ok(int dtype) { return dtype == TOPMOE_DTYPE_FP32 || dtype == TOPMOE_DTYPE_BF16; }

int elem_bytes(int dtype) { return dtype == TOPMOE_DTYPE_FP32 ? 4 : 2; }

struct Cand {
  GemmShape sh;
  double tflops;  // measured sustained rate of the whole chip with this shape (MI355X)
  int per_cu;     // blocks resident per CU (LDS / registers)
};

// Pick the launch shape minimising rounds x (tile time + fixed per-tile
// cost), with the tile time from the shape's measured sustained rate.
// Tiles: M tiles over `groups` groups x ceil(Nout / BN).
GemmShape choose(const Cand* cands, int n, int64_t M, int64_t Nout, int64_t K, int groups,
                 int nmat) {
  constexpr double kTileOverheadUs = 3.0;  // prologue fill + epilogue, measured order
  GemmShape best = cands[n - 1].sh;
  double best_cost = -1.0;
  for (int i = 0; i < n; ++i) {
    const GemmShape& c = cands[i].sh;
    const int64_t mt = grouped_mtiles_bound(M, groups, c.bm);
    const int64_t nt = (Nout + c.bn - 1) / c.bn;
    const int64_t tiles = mt * nt;
    if (tiles <= 0) continue;
    const int64_t slots = 256 * int64_t(cands[i].per_cu);
    const int64_t rounds = (tiles + slots - 1) / slots;
    const double tile_flop = 2.0 * nmat * c.bm * c.bn * double(K);
    const double slot_tflops = cands[i].tflops / double(slots);
    const double cost = double(rounds) * (tile_flop / (slot_tflops * 1e6) + kTileOverheadUs);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

// ---- launch-shape overrides (tuning sweeps, tests).  One slot per GEMM of
// the path; each holds "none", a shape, or "invalid" (an environment value
// that is not an instantiated shape: every plan that would use it fails).
constexpr int kSlots = 6;
const char* const kSlotEnv[kSlots] = {"TOPMOE_GATEUP_TILE", "TOPMOE_DOWN_TILE",
                                      "TOPMOE_BWDGU_TILE", "TOPMOE_BWDDH_TILE",
                                      "TOPMOE_WGU_TILE", "TOPMOE_WD_TILE"};
const int kSlotKind[kSlots] = {KIND_GATEUP, KIND_DOWN_Y, KIND_BWD_GU, KIND_BWD_DH, KIND_WGRAD2,
                               KIND_WGRAD1};

struct Override {
  int state = 0;  // 0 none, 1 shape, -1 invalid
  GemmShape sh;
};

struct Overrides {
  std::mutex mu;
  bool env_read = false;
  Override slot[kSlots];
};

Overrides& overrides() {
  static Overrides o;
  return o;
}

bool parse_shape(const char* v, GemmShape* out) {
  GemmShape g;
  char tail = 0;
  if (std::sscanf(v, "%dx%dx%dx%dx%dx%d%c", &g.bm, &g.bn, &g.wm, &g.wn, &g.rb, &g.stages,
                  &tail) != 6)
    return false;
  *out = g;
  return true;
}

// The override of a slot for `dtype`: TOPMOE_OK with *sh replaced when one is
// set, TOPMOE_ERR_BAD_ARG when the one set is not an instantiated shape for
// this GEMM and dtype.  The environment is read once, at the first call.
int apply_override(int slot, int dtype, GemmShape* sh) {
  Overrides& o = overrides();
  std::lock_guard<std::mutex> lock(o.mu);
  if (!o.env_read) {
    o.env_read = true;
    for (int i = 0; i < kSlots; ++i) {
      const char* v = std::getenv(kSlotEnv[i]);
      if (!v || !*v) continue;
      GemmShape g;
      o.slot[i].state = parse_shape(v, &g) ? 1 : -1;
      o.slot[i].sh = g;
    }
  }
  const Override& ov = o.slot[slot];
  if (ov.state == 0) return TOPMOE_OK;
  if (ov.state < 0 || !gemm_shape_supported(kSlotKind[slot], dtype, ov.sh))
    return TOPMOE_ERR_BAD_ARG;
  *sh = ov.sh;
  return TOPMOE_OK;
}

// Launch-shape tables: rates measured on MI355X over the dense bf16
// 16384 x 2048 x 6464 projections (sustained whole-chip TFLOP/s).  All are
// 8-wavefront tiles with 128-byte LDS rows: a direct-to-LDS load of 64-byte
// row pieces touches half of each 128-byte cache line and moves about half
// the bytes per clock (measured 32 against 59 B/clk/CU from L2).
const Cand kGateupBf16[] = {
    {{256, 128, 4, 2, 128, 2}, 1146.0, 1},
    {{128, 128, 2, 4, 128, 3}, 1056.0, 1},
    {{256, 64, 4, 2, 128, 3}, 1033.0, 1},
};
const Cand kDownBf16[] = {
    {{256, 256, 4, 2, 128, 2}, 1140.0, 1},
    {{256, 128, 4, 2, 128, 3}, 1093.0, 1},
    {{256, 256, 4, 2, 64, 4}, 1025.0, 1},
    {{128, 128, 2, 4, 128, 3}, 893.0, 1},
    {{256, 64, 4, 2, 128, 3}, 786.0, 1},
};
const Cand kFp32[] = {
    {{128, 64, 2, 2, 128, 2}, 100.0, 2},
    {{64, 64, 2, 2, 128, 3}, 90.0, 2},
};

// Few rows per group and long K: the projection streams weights from HBM.
// MFMA work is then nearly free; what counts is the weight bytes in flight
// per CU.  The 8-wavefront tiles with 128-byte rows carry the most; with at
// most 32 rows per expert a 64-row tile wastes less of each slice on clamped
// duplicate x rows than a 128-row one (measured cold on the 32-token decode
// step: gate/up 43.6 us against 45.3 us with 128 x 128; down 18.9 against
// 22.4 us, the down tile's smaller LDS slice also fitting two blocks per CU).
bool weight_streaming(int64_t M, int groups) { return M <= int64_t(groups) * 32; }

}  // namespace

GemmShape choose_gateup_tile(int64_t M, int64_t Nout, int64_t K, int groups, int dtype) {
  if (dtype == TOPMOE_DTYPE_FP32) return choose(kFp32, 2, M, Nout, K, groups, 2);
  return weight_streaming(M, groups) ? GemmShape{64, 128, 2, 4, 128, 3}
                                     : choose(kGateupBf16, 3, M, Nout, K, groups, 2);
}

GemmShape choose_down_tile(int64_t M, int64_t Nout, int64_t K, int groups, int dtype) {
  if (dtype == TOPMOE_DTYPE_FP32) return choose(kFp32, 2, M, Nout, K, groups, 1);
  return weight_streaming(M, groups) ? GemmShape{64, 128, 2, 4, 128, 3}
                                     : choose(kDownBf16, 5, M, Nout, K, groups, 1);
}

// ---- backward launch shapes (bf16 candidates measured on MI355X; fp32 the
// register-light tiles).
GemmShape gu_tile(int dtype) {
  return dtype == TOPMOE_DTYPE_FP32 ? GemmShape{128, 64, 2, 2, 128, 2}
                                    : GemmShape{256, 128, 4, 2, 128, 2};
}
GemmShape dh_tile(int dtype) {
  return dtype == TOPMOE_DTYPE_FP32 ? GemmShape{64, 64, 2, 2, 128, 3}
                                    : GemmShape{128, 128, 2, 4, 128, 3};
}
GemmShape wgu_tile(int dtype) {
  return dtype == TOPMOE_DTYPE_FP32 ? GemmShape{128, 64, 2, 2, 128, 2}
                                    : GemmShape{128, 256, 2, 4, 128, 2};
}
GemmShape wd_tile(int dtype) {
  return dtype == TOPMOE_DTYPE_FP32 ? GemmShape{128, 64, 2, 2, 128, 2}
                                    : GemmShape{256, 128, 4, 2, 128, 3};
}

int set_tile_override(int slot, const int* shape) {
  if (slot < 0 || slot >= kSlots) return TOPMOE_ERR_BAD_ARG;
  Overrides& o = overrides();
  std::lock_guard<std::mutex> lock(o.mu);
  o.env_read = true;  // an explicit setting replaces what the environment said
  if (shape == nullptr) {
    o.slot[slot].state = 0;
    return TOPMOE_OK;
  }
  const GemmShape g{shape[0], shape[1], shape[2], shape[3], shape[4], shape[5]};
  if (!gemm_shape_supported(kSlotKind[slot], TOPMOE_DTYPE_BF16, g) &&
      !gemm_shape_supported(kSlotKind[slot], TOPMOE_DTYPE_FP32, g))
    return TOPMOE_ERR_BAD_ARG;
  o.slot[slot].state = 1;
  o.slot[slot].sh = g;
  return TOPMOE_OK;
}

void choose_down_split(int64_t tiles, int64_t K, int elem, const GemmShape& sh, int* ksplit,
                       int* kchunk) {
  const int64_t kt = K * elem / sh.rb;  // K slices
  *ksplit = 1;
  *kchunk = int(kt);
  // Few output tiles and a long K (the 100-token fp32 FFN: 24 tiles, 76
  // slices): the tiles' K loops run one after another on a few CUs while the
  // others idle.  Chunks of K fill the CUs, and a small kernel adds the chunks'
  // fp32 partial sums in order and applies the epilogue.
  if (tiles <= 0 || tiles >= 128 || kt < 8) return;
  int64_t want = (256 + tiles - 1) / tiles;
  if (want > kt / 4) want = kt / 4;
  if (want > kMaxDownSplit) want = kMaxDownSplit;  // measured: more chunks of few slices each stream slower
  if (want < 2) return;
  const int64_t cs = (kt + want - 1) / want;
  *kchunk = int(cs);
  *ksplit = int((kt + cs - 1) / cs);  // every chunk non-empty
}

int plan_ffn(int64_t N, int64_t H, int64_t I, int dtype, FfnPlan* p) {
  if (!dtype_ok(dtype)) return TOPMOE_ERR_UNSUPPORTED_DTYPE;
  if (N < 0 || H < 64 || I < 64 || H % 64 || I % 64) return TOPMOE_ERR_BAD_SHAPE;
  const int el = elem_bytes(dtype);
  if (N > kMaxRows || !operand_ok(N, H, el) || !operand_ok(N, I, el) || !operand_ok(I, H, el))
    return TOPMOE_ERR_BAD_SHAPE;
  FfnPlan q;
  q.N = N; q.H = H; q.I = I; q.dtype = dtype; q.elem = elem_bytes(dtype);
  q.up = choose_gateup_tile(N, I, H, 1, dtype);
  q.down = choose_down_tile(N, H, I, 1, dtype);
  int st = apply_override(0, dtype, &q.up);
  if (st == TOPMOE_OK) st = apply_override(1, dtype, &q.down);
  if (st != TOPMOE_OK) return st;
  choose_down_split((N + q.down.bm - 1) / q.down.bm * ((H + q.down.bn - 1) / q.down.bn), I,
                    q.elem, q.down, &q.down_ksplit, &q.down_kchunk);
  q.off_h = 0;
  size_t o = align_up(size_t(N) * size_t(I) * q.elem);
  q.off_partial = o;
  if (q.down_ksplit > 1) o = align_up(o + size_t(q.down_ksplit) * size_t(N) * size_t(H) * 4);
  q.total = o == 0 ? kAlign : o;
  *p = q;
  return TOPMOE_OK;
}

int plan_moe(int64_t N, int64_t H, int64_t I, int E, int k, int dtype, MoePlan* p) {
  if (!dtype_ok(dtype)) return TOPMOE_ERR_UNSUPPORTED_DTYPE;
  if (N < 0 || H < 64 || I < 64 || H % 64 || I % 64) return TOPMOE_ERR_BAD_SHAPE;
  if (E < 1 || E > 64 || k < 1 || k > E) return TOPMOE_ERR_BAD_SHAPE;
  const int64_t rows = N * k;
  const int el = elem_bytes(dtype);
  if (rows > kMaxRows || !operand_ok(N, H, el) || !operand_ok(rows, I, el) ||
      !operand_ok(I, H, el))
    return TOPMOE_ERR_BAD_SHAPE;
  MoePlan q;
  q.N = N; q.H = H; q.I = I; q.E = E; q.k = k; q.dtype = dtype; q.elem = elem_bytes(dtype);
  q.rows = rows;
  // Router.  With W_router small enough for LDS (<= 64 KB, so two blocks
  // share a CU) and enough tokens, one-wavefront blocks copy it once and
  // route 16 tokens per pass (four lanes per token); about 1024 blocks of
  // whole passes.  With few tokens (decode) or a large W_router, one token
  // per 4-wavefront block, H split over the wavefronts.
  int ep = 1;
  while (ep < E) ep *= 2;
  const bool lds_fits = int64_t(ep) * H * 4 <= 64 * 1024;
  // With H a multiple of 16 loads (16 bytes each), 16 lanes per token in
  // four-wavefront blocks (mode 2): four times the wavefronts for the same
  // blocks.
  const bool p16 = H % (16 * (16 / q.elem)) == 0;
  q.router_mode = (lds_fits && N >= 256) ? (p16 ? 2 : 0) : 1;
  int64_t tb = 1;
  if (q.router_mode != 1) {
    const int64_t passes = (N + 15) / 16;
    tb = 16 * ((passes + 1023) / 1024);
  }
  // the permutation kernel stages E * blocks counts in LDS: at most 8192
  while (N > 0 && ((N + tb - 1) / tb) * E > 8192) tb *= 2;
  q.tb = int(tb);
  q.nblk = int((N + tb - 1) / tb);
  q.up = choose_gateup_tile(rows, I, H, E, dtype);
  q.down = choose_down_tile(rows, H, I, E, dtype);
  int st = apply_override(0, dtype, &q.up);
  if (st == TOPMOE_OK) st = apply_override(1, dtype, &q.down);
  if (st != TOPMOE_OK) return st;
  q.up_mtiles = grouped_mtiles_bound(rows, E, q.up.bm);
  q.down_mtiles = grouped_mtiles_bound(rows, E, q.down.bm);
  size_t o = 0;
  const size_t nbe = size_t(q.nblk) * size_t(E);
  q.off_count_part = o; o = align_up(o + nbe * 4);
  q.off_psum_part = o;  o = align_up(o + nbe * 4);
  q.off_offsets = o;    o = align_up(o + size_t(E + 1) * 4);
  q.off_counts_off = o; o = align_up(o + size_t(E + 1) * 4);
  q.off_zpart = o;      o = align_up(o + size_t(q.nblk) * 4);
  q.off_keep = o;       o = align_up(o + size_t(rows));
  q.off_sorted = o;     o = align_up(o + size_t(rows) * 4);
  q.off_alpha_g = o;    o = align_up(o + size_t(rows) * 4);
  choose_down_split(q.down_mtiles * ((H + q.down.bn - 1) / q.down.bn), I, q.elem, q.down,
                    &q.down_ksplit, &q.down_kchunk);
  // the 64 x 128 tiles of eight wavefronts carry the in-block routing (one
  // entry per thread)
  const bool streaming64 = q.up.bm == 64 && q.up.bn == 128 && q.down.bm == 64 &&
                           q.down.bn == 128 && q.up.wm * q.up.wn * 64 >= kInlineMaxEntries &&
                           q.down.wm * q.down.wn * 64 >= kInlineMaxEntries;
  q.inline_ok = rows <= kInlineMaxEntries && streaming64 && q.down_ksplit <= 1;
  // Every token against every expert only while that costs no MFMA time
  // (one row tile per expert) and the tiles and router blocks of the launch
  // fit on the chip's 256 CUs at once (the router blocks are the launch's
  // last: they must not wait for tiles to finish).
  const int64_t up_tiles_allx = int64_t(E) * ((I + q.up.bn - 1) / q.up.bn);
  q.allx = q.inline_ok && q.router_mode == 1 && q.tb == 1 && E <= 16 && N <= q.up.bm &&
           up_tiles_allx + q.nblk <= 256;
  const int64_t h_rows = q.allx && int64_t(E) * N > rows ? int64_t(E) * N : rows;
  q.off_h = o;          o = align_up(o + size_t(h_rows) * size_t(I) * q.elem);
  q.off_slots = o;  // k-slots (k >= 2 only: with k = 1 the down GEMM writes y itself)
  if (k > 1) o = align_up(o + size_t(rows) * size_t(H) * q.elem);
  q.off_partial = o;
  if (q.down_ksplit > 1) o = align_up(o + size_t(q.down_ksplit) * size_t(rows) * size_t(H) * 4);
  q.total = o == 0 ? kAlign : o;
  *p = q;
  return TOPMOE_OK;
}

int plan_ffn_bwd(int64_t N, int64_t H, int64_t I, int dtype, FfnBwdPlan* p) {
  FfnPlan f;
  const int st = plan_ffn(N, H, I, dtype, &f);
  if (st != TOPMOE_OK) return st;
  const int el = f.elem;
  FfnBwdPlan q;
  q.N = N; q.H = H; q.I = I; q.dtype = dtype; q.elem = el;
  q.ldk = (N + 63) / 64 * 64;
  if (!operand_ok(N, 2 * I, el) || !operand_ok(H, 2 * I, el) || !operand_ok(I, q.ldk, el) ||
      !operand_ok(H, q.ldk, el))
    return TOPMOE_ERR_BAD_SHAPE;
  q.gu = gu_tile(dtype);
  q.dh = dh_tile(dtype);
  q.dx = choose_down_tile(N, H, 2 * I, 1, dtype);
  q.wgu = wgu_tile(dtype);
  q.wd = wd_tile(dtype);
  {
    GemmShape* sh[5] = {&q.gu, &q.dh, &q.dx, &q.wgu, &q.wd};
    const int slot[5] = {2, 3, 1, 4, 5};
    for (int i = 0; i < 5; ++i) {
      const int so = apply_override(slot[i], dtype, sh[i]);
      if (so != TOPMOE_OK) return so;
    }
  }
  const size_t e = size_t(el);
  size_t o = 0;
  q.off_wgT = o;  o = align_up(o + size_t(H) * size_t(2 * I) * e);
  q.off_wdT = o;  o = align_up(o + size_t(I) * size_t(H) * e);
  q.off_xT = o;   o = align_up(o + size_t(H) * size_t(q.ldk) * e);
  q.off_dyT = o;  o = align_up(o + size_t(H) * size_t(q.ldk) * e);
  q.off_gu = o;   o = align_up(o + size_t(N) * size_t(I) * 2 * e);
  q.off_dgdu = o; o = align_up(o + size_t(N) * size_t(2 * I) * e);
  q.off_dgT = o;  o = align_up(o + size_t(I) * size_t(q.ldk) * e);
  q.off_duT = o;  o = align_up(o + size_t(I) * size_t(q.ldk) * e);
  q.off_hT = o;   o = align_up(o + size_t(I) * size_t(q.ldk) * e);
  q.total = o;
  *p = q;
  return TOPMOE_OK;
}

int plan_moe_bwd(int64_t N, int64_t H, int64_t I, int E, int k, int dtype, MoeBwdPlan* p) {
  MoePlan r;
  const int st = plan_moe(N, H, I, E, k, dtype, &r);
  if (st != TOPMOE_OK) return st;
  const int el = r.elem;
  const int64_t rows = r.rows;
  MoeBwdPlan q;
  q.route = r;
  // every group's rows rounded up to 64: at most 63 extra per group
  q.ldk = (rows + 63) / 64 * 64 + 64 * int64_t(E);
  if (!operand_ok(rows, 2 * I, el) || !operand_ok(H, 2 * I, el) || !operand_ok(I, q.ldk, el) ||
      !operand_ok(H, q.ldk, el) || q.ldk > kMaxRows)
    return TOPMOE_ERR_BAD_SHAPE;
  q.gu = gu_tile(dtype);
  q.dh = dh_tile(dtype);
  q.dx = choose_down_tile(rows, H, 2 * I, E, dtype);
  q.wgu = wgu_tile(dtype);
  q.wd = wd_tile(dtype);
  {
    GemmShape* sh[5] = {&q.gu, &q.dh, &q.dx, &q.wgu, &q.wd};
    const int slot[5] = {2, 3, 1, 4, 5};
    for (int i = 0; i < 5; ++i) {
      const int so = apply_override(slot[i], dtype, sh[i]);
      if (so != TOPMOE_OK) return so;
    }
  }
  q.gu_mtiles = grouped_mtiles_bound(rows, E, q.gu.bm);
  q.dh_mtiles = grouped_mtiles_bound(rows, E, q.dh.bm);
  q.dx_mtiles = grouped_mtiles_bound(rows, E, q.dx.bm);
  q.nt_h = int((I + q.dh.bn - 1) / q.dh.bn);
  q.nchunk = int((N + kDwrChunk - 1) / kDwrChunk);
  const size_t e = size_t(el);
  // routing buffers first (the forward's own layout), then the backward's
  size_t o = r.off_h;
  q.off_probs = o; o = align_up(o + size_t(N) * size_t(E) * 4);
  q.off_lse = o;   o = align_up(o + size_t(N) * 4);
  q.off_topk = o;  o = align_up(o + size_t(rows) * 4);
  q.off_alpha = o; o = align_up(o + size_t(rows) * 4);
  q.off_aux = o;   o = align_up(o + 4);
  q.off_wgT = o;   o = align_up(o + size_t(E) * size_t(H) * size_t(2 * I) * e);
  q.off_wdT = o;   o = align_up(o + size_t(E) * size_t(I) * size_t(H) * e);
  q.off_xT = o;    o = align_up(o + size_t(H) * size_t(q.ldk) * e);
  q.off_dyT = o;   o = align_up(o + size_t(H) * size_t(q.ldk) * e);
  q.off_gu = o;    o = align_up(o + size_t(rows) * size_t(I) * 2 * e);
  q.off_dgdu = o;  o = align_up(o + size_t(rows) * size_t(2 * I) * e);
  q.off_dgT = o;   o = align_up(o + size_t(I) * size_t(q.ldk) * e);
  q.off_duT = o;   o = align_up(o + size_t(I) * size_t(q.ldk) * e);
  q.off_hT = o;    o = align_up(o + size_t(I) * size_t(q.ldk) * e);
  q.off_dal = o;   o = align_up(o + size_t(rows) * size_t(q.nt_h) * 4);
  q.off_slots = o; o = align_up(o + size_t(rows) * size_t(H) * e);
  q.off_dr = o;    o = align_up(o + size_t(N) * size_t(E) * 4);
  q.off_dwr = o;   o = align_up(o + size_t(q.nchunk) * size_t(E) * size_t(H) * 4);
  q.total = o;
  *p = q;
  return TOPMOE_OK;
}

}  // namespace topmoe
