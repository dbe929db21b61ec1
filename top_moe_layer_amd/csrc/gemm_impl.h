// Grouped MFMA GEMM for the three FFN projections (gfx950, wave64).
//
// Every projection is nn.Linear(in, out, bias=False) applied to token rows
// (MiniMind lesson 13, section 3 step 3; section 0 equations): out = A W^T with
// A [rows, K] and W [Nout, K], both contiguous along K.  For the MoE each
// expert's rows form one group (the per-expert token lists of walkthrough
// step 5); the kernel walks a flattened list of (group, row-tile) x column-tile
// work items whose group boundaries it reads from the device-side expert
// offsets, so no host synchronisation is needed.
//
// Block: 256 threads = 4 wavefronts in a 2 x 2 arrangement; block tile BM x BN
// of every output matrix (two matrices, gate and up, for the first
// projection), K stepped by one 128-byte row chunk (64 bf16 or 32 fp32).
// Operands are staged global -> registers -> LDS with double buffering; the
// 128-byte LDS rows keep their eight 16-byte chunks XOR-swizzled by (row & 7)
// so the 16-byte fragment reads of a wavefront are bank-conflict free.
// MFMA: v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32 (fp32),
// fp32 accumulation.
//
// Epilogues:
//   gate/up : h = SiLU(g) * u = g * u / (1 + e^-g)  (lesson 13, section 1.2),
//             stored in the operand dtype in grouped row order;
//   down    : o * alpha_{t,j} (the renormalised router weight; 1 for the dense
//             FFN), written to y[t] (k == 1 or dense) or to the fp32 slot of
//             entry (t, j) (k >= 2) for the fixed-order combine.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace topmoe {

template <typename T>
struct Mfma;

template <>
struct Mfma<bf16_t> {
  static constexpr int BK = 64;  // elements per 128-byte row chunk
  __device__ static __forceinline__ void mma(f32x16& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// fp32: each 16-byte fragment holds 4 consecutive k of one lane group; the two
// lane groups (lanes 0-31, 32-63) cover k = 8q + s and 8q + 4 + s.  A and B use
// the same assignment, so the 4 depth-2 MFMAs sum all 8 k of the step.
template <>
struct Mfma<float> {
  static constexpr int BK = 32;
  __device__ static __forceinline__ void mma(f32x16& c, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s]), __uint_as_float(b[s]), c,
                                               0, 0, 0);
  }
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  // g * u / (1 + 2^(-g log2 e)); v_exp_f32 and v_rcp_f32 (about 1 ulp each)
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

template <typename T, int BM, int BN, int KIND>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmParams p) {
  constexpr int NB = KIND == KIND_GATEUP ? 2 : 1;
  constexpr int TM = BM / 64, TN = BN / 64;  // 32x32 MFMA tiles per wavefront
  constexpr int AR = BM / 32, BR = BN / 32;  // 16-byte loads per thread per operand
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int STAGE = A_BYTES + NB * B_BYTES;
  static_assert(TM >= 1 && TN >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ int s_tile[3];

  const int tid = threadIdx.x;
  const int nt_count = (p.Nout + BN - 1) / BN;
  const int nt = int(blockIdx.x % unsigned(nt_count));
  const int mt = int(blockIdx.x / unsigned(nt_count));

  // ---- which group (expert) and rows this tile covers
  int e = 0;
  int64_t row0;
  int rows;
  if (p.offsets == nullptr) {
    row0 = int64_t(mt) * BM;
    const int64_t left = p.M - row0;
    rows = left < BM ? int(left) : BM;
  } else {
    if (tid < 64) {
      const int lane = tid;
      int off = 0, c = 0;
      if (lane < p.E) {
        off = p.offsets[lane];
        c = p.offsets[lane + 1] - off;
      }
      const int tiles = (c + BM - 1) / BM;
      const int incl = wave_inclusive_scan(tiles, lane);
      const uint64_t before = __ballot(lane < p.E && incl <= mt);
      const int ge = __popcll(before);
      if (lane == 0) s_tile[0] = ge;
      if (lane == ge && ge < p.E) {
        const int local = mt - (incl - tiles);
        s_tile[1] = off + local * BM;
        const int left = c - local * BM;
        s_tile[2] = left < BM ? left : BM;
      }
    }
    __syncthreads();
    e = s_tile[0];
    if (e >= p.E) return;  // past the last tile: the whole block leaves
    row0 = s_tile[1];
    rows = s_tile[2];
  }
  if (rows <= 0) return;

  // ---- global source addresses (rows clamped into the valid range)
  const int lc = tid & 7, lr = tid >> 3;
  const char* a_src[AR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    const int r = lr + 32 * i;
    const int64_t gr = row0 + (r < rows ? r : rows - 1);
    int64_t arow = gr;
    if (KIND == KIND_GATEUP && p.entries != nullptr) arow = p.entries[gr] / p.k;
    a_src[i] = static_cast<const char*>(p.A) + (arow * p.K) * int64_t(sizeof(T)) + lc * 16;
  }
  const int n0 = nt * BN;
  const char* b_src[NB][BR];
#pragma unroll
  for (int i = 0; i < BR; ++i) {
    int n = n0 + lr + 32 * i;
    n = n < p.Nout ? n : p.Nout - 1;
    const int64_t off = ((int64_t(e) * p.Nout + n) * p.K) * int64_t(sizeof(T)) + lc * 16;
    b_src[0][i] = static_cast<const char*>(p.B0) + off;
    if (NB == 2) b_src[NB - 1][i] = static_cast<const char*>(p.B1) + off;
  }
  const int w_off = lr * 128 + ((lc ^ (lr & 7)) << 4);

  u32x4 ra[AR], rb[NB][BR];
  auto gload = [&](int kt) {
    const int64_t ko = int64_t(kt) * 128;
#pragma unroll
    for (int i = 0; i < AR; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + ko);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < BR; ++i) rb[b][i] = *reinterpret_cast<const u32x4*>(b_src[b][i] + ko);
  };
  auto lstore = [&](int stage) {
    char* s = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < AR; ++i) *reinterpret_cast<u32x4*>(s + w_off + i * 4096) = ra[i];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < BR; ++i)
        *reinterpret_cast<u32x4*>(s + A_BYTES + b * B_BYTES + w_off + i * 4096) = rb[b][i];
  };

  const int KT = p.K / Mfma<T>::BK;
  gload(0);
  lstore(0);
  __syncthreads();

  f32x16 acc[NB][TM][TN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.f;

  const int wid = tid >> 6, lane = tid & 63;
  const int fr = lane & 31, fg = lane >> 5;
  const int wm = (wid >> 1) * (BM / 2), wn = (wid & 1) * (BN / 2);

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const char* sA = smem + cur * STAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rd = ((2 * q + fg) ^ (fr & 7)) << 4;
      u32x4 af[TM], bfr[NB][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(sA + (wm + 32 * i + fr) * 128 + rd);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[b][j] = *reinterpret_cast<const u32x4*>(sA + A_BYTES + b * B_BYTES +
                                                      (wn + 32 * j + fr) * 128 + rd);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) Mfma<T>::mma(acc[b][i][j], af[i], bfr[b][j]);
    }
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  32x32 accumulator layout: lane (fr, fg), register v holds
  // row 8*(v/4) + 4*fg + v%4, column fr of the MFMA tile.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm + 32 * i + 8 * (v >> 2) + 4 * fg + (v & 3);
      if (r >= rows) continue;
      const int64_t grow = row0 + r;
      if (KIND == KIND_GATEUP) {
        T* out = static_cast<T*>(p.out) + grow * p.Nout;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn + 32 * j + fr;
          if (col < p.Nout) out[col] = from_f32<T>(silu_mul(acc[0][i][j][v], acc[NB - 1][i][j][v]));
        }
      } else {
        const int64_t ent = p.entries != nullptr ? int64_t(p.entries[grow]) : grow;
        const float a = p.alpha != nullptr ? p.alpha[ent] : 1.0f;
        if (KIND == KIND_DOWN_Y) {
          T* out = static_cast<T*>(p.out) + (ent / p.k) * p.Nout;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn + 32 * j + fr;
            if (col < p.Nout) out[col] = from_f32<T>(acc[0][i][j][v] * a);
          }
        } else {
          float* out = static_cast<float*>(p.out) + ent * p.Nout;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn + 32 * j + fr;
            if (col < p.Nout) out[col] = acc[0][i][j][v] * a;
          }
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int KIND>
hipError_t launch_gemm_t(const GemmParams& p, int64_t mtiles, hipStream_t s) {
  const int64_t nt = (p.Nout + BN - 1) / BN;
  const int64_t grid = mtiles * nt;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, KIND>), dim3(unsigned(grid)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T, int KIND>
hipError_t launch_gemm_tiles(GemmShape sh, const GemmParams& p, int64_t mtiles, hipStream_t s) {
  if (sh.bm == 256 && sh.bn == 128) return launch_gemm_t<T, 256, 128, KIND>(p, mtiles, s);
  if (sh.bm == 128 && sh.bn == 128) return launch_gemm_t<T, 128, 128, KIND>(p, mtiles, s);
  if (sh.bm == 128 && sh.bn == 64) return launch_gemm_t<T, 128, 64, KIND>(p, mtiles, s);
  if (sh.bm == 64 && sh.bn == 64) return launch_gemm_t<T, 64, 64, KIND>(p, mtiles, s);
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_gemm_dtype(int kind, GemmShape sh, const GemmParams& p, int64_t mtiles,
                             hipStream_t s) {
  switch (kind) {
    case KIND_GATEUP: return launch_gemm_tiles<T, KIND_GATEUP>(sh, p, mtiles, s);
    case KIND_DOWN_Y: return launch_gemm_tiles<T, KIND_DOWN_Y>(sh, p, mtiles, s);
    case KIND_DOWN_SLOTS: return launch_gemm_tiles<T, KIND_DOWN_SLOTS>(sh, p, mtiles, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace topmoe
