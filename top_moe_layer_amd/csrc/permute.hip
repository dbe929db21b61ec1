// Token permutation, load-balancing loss and the k-slot combine.
//
// The MoE dispatch of MiniMind lesson 13, walkthrough step 5 visits experts in
// ascending id and, for each, the tokens that selected it in ascending token
// order (mask / nonzero), runs the expert on those rows and adds the weighted
// rows back with index_add_.  Here the same grouping is built once, without a
// host round trip:
//   * permute: per-expert totals c_e and their exclusive prefix sum (expert
//     offsets), the aux loss aux = E * coef * sum_e (c_e / N) * (sum_t p_{t,e} / N)
//     (lesson 13, section 1.6 equation; walkthrough step 6), and a stable
//     scatter of the entries (t, j) in t*k + j order into expert groups, so
//     each group lists its tokens in ascending order (with each entry's alpha
//     copied beside it for the down projection's epilogue);
//   * combine: y_t = sum of the k alpha-scaled expert rows (each in the output
//     dtype) in ascending expert id, accumulated in fp32 and rounded once.
// With an expert capacity C (the study notes' section 10 names it; the
// standard form is a reading: each expert keeps the first C of its entries in
// the dispatch order, i.e. ascending token), the scatter keeps an entry only
// if its rank within its expert is below C: the expert groups, the offsets and
// the token lists hold the kept entries (the lists end in -1), a flag per
// entry records the choice for the combine, and aux still counts every
// selection.  Block 0 also finishes the router z-loss from the router
// blocks' partial sums.
// All integer work is exact; the only float reductions run in a fixed order.
#include "device_common.h"
#include "kernels.h"

#include "../../include/topmoe.h"

namespace topmoe {

namespace {

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Offsets, aux loss and scatter in one launch.  count_part / psum_part are
// expert-major [E, nblk] (nblk router blocks, E * nblk <= 8192).  Scatter
// block s owns router blocks [s*G, s*G + G): it stages all counts in LDS,
// derives every expert's total and the count of entries in router blocks
// before its own, and so its base slot per expert; it then ranks its entries
// (t*k + j order) among equal experts with wavefront ballots.  Block 0 also
// writes the expert offsets and the aux loss (sums of p in a fixed order).
constexpr int kScanMax = 8192;

__global__ __launch_bounds__(256) void permute_kernel(
    const int32_t* __restrict__ count_part, const float* __restrict__ psum_part,
    const float* __restrict__ z_part, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ alpha, int nblk, int G, int E, int k, int tb, int64_t N,
    float coef, float z_coef, int cap, int32_t* __restrict__ offsets,
    int32_t* __restrict__ counts_off, float* __restrict__ aux, float* __restrict__ z_loss,
    int32_t* __restrict__ sorted_entry, float* __restrict__ alpha_g,
    int32_t* __restrict__ sorted_tok, uint8_t* __restrict__ keep,
    int32_t* __restrict__ topk_copy, float* __restrict__ alpha_copy,
    int32_t* __restrict__ offsets_copy) {
  __shared__ int s_c[kScanMax];
  __shared__ float s_p[kScanMax];  // block 0 only
  __shared__ int s_tot[64];
  __shared__ int s_base[64];   // the block's first rank within each expert
  __shared__ int s_koff[64];   // kept-entry offset of each expert
  __shared__ int s_ktot;
  __shared__ double s_ps[64];
  __shared__ int run[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool first = blockIdx.x == 0;
  const int total = E * nblk;
  const int bfirst = int(blockIdx.x) * G;
  // This block's entries: wavefront 0 fetches the first 64 now, so their
  // latency overlaps the staging below.
  const int64_t tok0 = int64_t(bfirst) * tb;
  const int64_t tok1 = tok0 + int64_t(G) * tb < N ? tok0 + int64_t(G) * tb : N;
  const int64_t e0 = tok0 * k, e1 = tok1 * k;
  int ex_first = -1;
  float al_first = 0.f;
  if (wave == 0 && e0 + lane < e1) {
    ex_first = topk_idx[e0 + lane];
    al_first = alpha[e0 + lane];
  }
  // All counts (and, in block 0, all sums of p), 8 loads per thread in flight.
  for (int base = 0; base < total; base += 256 * 8) {
    int c[8];
    float ps[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * 256 + tid;
      c[j] = i < total ? count_part[i] : 0;
      ps[j] = (first && i < total) ? psum_part[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * 256 + tid;
      if (i < total) {
        s_c[i] = c[j];
        if (first) s_p[i] = ps[j];
      }
    }
  }
  if (tid < 64) run[tid] = 0;
  __syncthreads();

  for (int e = wave; e < E; e += 4) {
    int tot = 0, pre = 0;
    double ps = 0.0;
    for (int b = lane; b < nblk; b += 64) {
      const int c = s_c[e * nblk + b];
      tot += c;
      pre += b < bfirst ? c : 0;
      if (first) ps += double(s_p[e * nblk + b]);
    }
    tot = wave_sum_int(tot);
    pre = wave_sum_int(pre);
    if (first) ps = wave_sum(ps);
    if (lane == 0) { s_tot[e] = tot; s_base[e] = pre; s_ps[e] = ps; }
  }
  __syncthreads();

  if (wave == 0) {
    const int c = lane < E ? s_tot[lane] : 0;
    const int kc = (cap > 0 && c > cap) ? cap : c;  // entries the expert keeps
    const int kincl = wave_inclusive_scan(kc, lane);
    if (lane < E) s_koff[lane] = kincl - kc;
    if (lane == E - 1) s_ktot = kincl;
    if (first) {
      if (lane < E) offsets[lane] = kincl - kc;
      if (lane == E - 1) offsets[E] = kincl;
      if (offsets_copy != nullptr) {
        if (lane < E) offsets_copy[lane] = kincl - kc;
        if (lane == E - 1) offsets_copy[E] = kincl;
      }
      if (counts_off != nullptr) {  // offsets of every selection (before any capacity)
        const int incl = wave_inclusive_scan(c, lane);
        if (lane < E) counts_off[lane] = incl - c;
        if (lane == E - 1) counts_off[E] = incl;
      }
      // aux = E * coef * sum_e c_e * (sum_t p_{t,e}) / N^2 (fixed summation order;
      // c_e counts every selection, kept or not)
      double term = lane < E ? double(c) * s_ps[lane] : 0.0;
      term = wave_sum(term);
      if (lane == 0) {
        float a = 0.f;
        if (coef != 0.f && N > 0) a = float(double(E) * double(coef) * term / (double(N) * double(N)));
        *aux = a;
      }
      // z-loss = z_coef * (sum of the router blocks' logsumexp^2 sums) / N
      if (z_loss != nullptr) {
        double z = 0.0;
        for (int b = lane; b < nblk; b += 64) z += double(z_part[b]);
        z = wave_sum(z);
        if (lane == 0) *z_loss = (z_coef != 0.f && N > 0) ? float(double(z_coef) * z / double(N)) : 0.f;
      }
    }
  }
  __syncthreads();
  if (first && sorted_tok != nullptr && cap > 0) {  // the lists end in -1 after the kept entries
    for (int64_t i = s_ktot + tid; i < N * k; i += 256) sorted_tok[i] = -1;
  }

  if (wave == 0) {
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int64_t base = e0; base < e1; base += 64) {
      const int64_t ent = base + lane;
      const bool valid = ent < e1;
      const int ex = base == e0 ? ex_first : valid ? topk_idx[ent] : -1;
      const float al = base == e0 ? al_first : valid ? alpha[ent] : 0.f;
      uint64_t peers = 0ull;  // lanes holding the same expert
      uint64_t todo = __ballot(valid);
      while (todo) {
        const int leader = __ffsll((long long)todo) - 1;
        const int le = __shfl(ex, leader, 64);
        const uint64_t m = __ballot(valid && ex == le);
        if (valid && ex == le) peers = m;
        todo &= ~m;
      }
      if (valid && topk_copy != nullptr) {
        topk_copy[ent] = ex;
        alpha_copy[ent] = al;
      }
      if (valid) {
        const int rank = s_base[ex] + run[ex] + __popcll(peers & lt_mask);  // within expert ex
        const bool kept = cap <= 0 || rank < cap;
        if (kept) {
          const int dest = s_koff[ex] + rank;
          sorted_entry[dest] = int32_t(ent);
          alpha_g[dest] = al;
          if (sorted_tok) sorted_tok[dest] = int32_t(ent / k);
        }
        if (keep) keep[ent] = kept ? 1 : 0;
      }
      __builtin_amdgcn_wave_barrier();
      if (valid && (peers & lt_mask) == 0ull) run[ex] += __popcll(peers);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// 16 bytes of the dtype (8 bf16 or 4 fp32 values) to / from fp32.
template <typename T>
struct Vec16 {
  static constexpr int n = 16 / int(sizeof(T));
};
template <typename T>
__device__ __forceinline__ void load16(const T* p, float (&v)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void load16<float>(const float* p, float (&v)[4]) {
  const f32x4 q = *reinterpret_cast<const f32x4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
template <>
__device__ __forceinline__ void load16<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(q[i] << 16);
    v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
  }
}
template <typename T>
__device__ __forceinline__ void store16(T* p, const float (&v)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void store16<float>(float* p, const float (&v)[4]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store16<bf16_t>(bf16_t* p, const float (&v)[8]) {
  u32x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    q[i] = uint32_t(f32_to_bf16(v[2 * i])) | (uint32_t(f32_to_bf16(v[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4*>(p) = q;
}

// y[t, 16 bytes] = residual (or 0) + the k slot rows of token t (each already
// rounded to the output dtype, like the terms the pages' index_add_
// accumulates), in ascending expert id, accumulated in fp32 and rounded once.
// The residual may alias y: each thread reads its residual piece before
// writing the same piece of y.  Without slots (k == 1 under a capacity, where
// the down GEMM wrote the kept tokens' rows of y) only the tokens whose entry
// was dropped are written: y = residual (or 0).  K2: k == 2 with slots, both
// slot pieces loaded at once (one memory latency after the ids, not two).
template <typename T, bool K2>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ slots,
                                                      const int32_t* __restrict__ topk_idx,
                                                      const uint8_t* __restrict__ keep,
                                                      const T* residual, int64_t N, int H, int k,
                                                      T* y) {
  constexpr int V = Vec16<T>::n;
  const int hv = H / V;  // H is a multiple of 64
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= N * hv) return;
  const int64_t t = gid / hv;
  const int h = int(gid - t * hv) * V;
  if (slots == nullptr && keep[t] != 0) return;  // kept: written by the down GEMM
  const int32_t* ids = topk_idx + t * k;
  float acc[V];
  if (residual != nullptr) {
    load16<T>(residual + t * H + h, acc);  // y starts from the residual stream
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
  }
  if constexpr (K2) {
    const int first = ids[1] < ids[0] ? 1 : 0;  // the lower expert id is added first
    const bool keep0 = keep == nullptr || keep[t * 2 + first] != 0;
    const bool keep1 = keep == nullptr || keep[t * 2 + (1 - first)] != 0;
    float v0[V], v1[V];
    load16<T>(slots + (t * 2 + first) * H + h, v0);
    load16<T>(slots + (t * 2 + (1 - first)) * H + h, v1);
    if (keep0) {
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += v0[i];
    }
    if (keep1) {
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += v1[i];
    }
    store16<T>(y + t * H + h, acc);
    return;
  }
  int prev = -1;
  for (int r = 0; r < k; ++r) {
    int best_j = 0, best_e = 1 << 30;
    for (int j = 0; j < k; ++j) {
      const int e = ids[j];
      if (e > prev && e < best_e) { best_e = e; best_j = j; }
    }
    prev = best_e;
    if (slots == nullptr) break;
    if (keep != nullptr && keep[t * k + best_j] == 0) continue;  // dropped by the capacity
    float v[V];
    load16<T>(slots + (t * k + best_j) * H + h, v);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += v[i];
  }
  store16<T>(y + t * H + h, acc);
}

// The down projection's epilogue over split-K partial sums (grouped row r,
// four columns per thread): the chunks' fp32 sums added in chunk order, then
// alpha, the entry's destination and the residual as in the GEMM's own
// epilogue, rounded once.
template <typename T, bool SLOTS>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float* __restrict__ partial, int ksplit, int64_t M, int Nout,
    const int32_t* __restrict__ offsets, int E, const int32_t* __restrict__ entries,
    const float* __restrict__ alpha, int k, const T* residual, T* out) {
  const int nq = Nout / 4;
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rows = offsets != nullptr ? int64_t(offsets[E]) : M;
  if (gid >= rows * nq) return;
  const int64_t r = gid / nq;
  const int c = int(gid - r * nq) * 4;
  const float a = alpha != nullptr ? alpha[r] : 1.f;
  const int64_t ent = entries != nullptr ? int64_t(entries[r]) : r;
  // the first kMaxDownSplit chunks' pieces all in flight at once, then added
  // in chunk order (a longer split, which the planner does not make, adds the
  // rest one by one)
  float v[kMaxDownSplit][4];
#pragma unroll
  for (int ch = 0; ch < kMaxDownSplit; ++ch)
    if (ch < ksplit) load4<float>(partial + (int64_t(ch) * M + r) * Nout + c, v[ch]);
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ch = 0; ch < kMaxDownSplit; ++ch)
    if (ch < ksplit) {
#pragma unroll
      for (int w = 0; w < 4; ++w) sum[w] += v[ch][w];
    }
  for (int ch = kMaxDownSplit; ch < ksplit; ++ch) {
    float u[4];
    load4<float>(partial + (int64_t(ch) * M + r) * Nout + c, u);
#pragma unroll
    for (int w = 0; w < 4; ++w) sum[w] += u[w];
  }
  float b[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) b[w] = sum[w] * a;
  if constexpr (SLOTS) {
    store4<T>(out + ent * Nout + c, b);
  } else {
    const int64_t o = (ent / k) * Nout + c;
    if (residual != nullptr) {
      float rr[4];
      load4<T>(residual + o, rr);
#pragma unroll
      for (int w = 0; w < 4; ++w) b[w] = rr[w] + b[w];
    }
    store4<T>(out + o, b);
  }
}

__global__ void empty_route_kernel(int E, int32_t* offsets, float* aux, float* z_loss) {
  const int tid = threadIdx.x;
  if (tid <= E) offsets[tid] = 0;
  if (tid == 0) *aux = 0.f;
  if (tid == 0 && z_loss != nullptr) *z_loss = 0.f;
}

}  // namespace

hipError_t launch_permute(const int32_t* count_part, const float* psum_part,
                          const float* z_part, const int32_t* topk_idx, const float* alpha,
                          int nblk, int E, int k, int tb, int64_t N, float coef, float z_coef,
                          int cap, int32_t* offsets, int32_t* counts_off, float* aux,
                          float* z_loss, int32_t* sorted_entry, float* alpha_g,
                          int32_t* sorted_tok, uint8_t* keep, int32_t* topk_copy,
                          float* alpha_copy, int32_t* offsets_copy, const Launch& s) {
  if (nblk <= 0) return hipSuccess;
  if (int64_t(E) * nblk > kScanMax) return hipErrorInvalidValue;
  const int G = nblk > 256 ? (nblk + 255) / 256 : 1;  // router blocks per scatter block
  const int nsb = (nblk + G - 1) / G;
  return launch_kernel(permute_kernel, dim3(nsb), dim3(256), 0, s, count_part, psum_part, z_part,
                       topk_idx, alpha, nblk, G, E, k, tb, N, coef, z_coef, cap, offsets,
                       counts_off, aux, z_loss, sorted_entry, alpha_g, sorted_tok, keep,
                       topk_copy, alpha_copy, offsets_copy);
}

hipError_t launch_combine(const void* slots, const int32_t* topk_idx, const uint8_t* keep,
                          const void* residual, int64_t N, int H, int k, int dtype, void* y,
                          const Launch& s) {
  const int64_t work = N * (H / (dtype == TOPMOE_DTYPE_FP32 ? 4 : 8));  // 16-byte pieces
  if (work <= 0) return hipSuccess;
  const int64_t grid = (work + 255) / 256;
  const bool k2 = slots != nullptr && k == 2;
#define TOPMOE_COMBINE(T, K2)                                                                \
  return launch_kernel(combine_kernel<T, K2>, dim3(grid), dim3(256), 0, s,                   \
                       static_cast<const T*>(slots), topk_idx, keep,                         \
                       static_cast<const T*>(residual), N, H, k, static_cast<T*>(y))
  if (dtype == TOPMOE_DTYPE_FP32) {
    if (k2) TOPMOE_COMBINE(float, true);
    TOPMOE_COMBINE(float, false);
  }
  if (k2) TOPMOE_COMBINE(bf16_t, true);
  TOPMOE_COMBINE(bf16_t, false);
#undef TOPMOE_COMBINE
}

hipError_t launch_splitk_reduce(const float* partial, int ksplit, int64_t M, int Nout,
                                const int32_t* offsets, int E, const int32_t* entries,
                                const float* alpha, int k, const void* residual, int dtype,
                                bool slots, void* out, const Launch& s) {
  const int64_t work = M * (Nout / 4);
  if (work <= 0) return hipSuccess;
  const dim3 grid(unsigned((work + 255) / 256));
#define TOPMOE_RED(T, SL)                                                                   \
  return launch_kernel(splitk_reduce_kernel<T, SL>, grid, dim3(256), 0, s, partial, ksplit, M, \
                       Nout, offsets, E, entries, alpha, k, static_cast<const T*>(residual),  \
                       static_cast<T*>(out))
  if (dtype == TOPMOE_DTYPE_FP32) {
    if (slots) TOPMOE_RED(float, true);
    TOPMOE_RED(float, false);
  }
  if (slots) TOPMOE_RED(bf16_t, true);
  TOPMOE_RED(bf16_t, false);
#undef TOPMOE_RED
}

hipError_t launch_empty_route(int E, int32_t* offsets, float* aux, float* z_loss,
                              const Launch& s) {
  return launch_kernel(empty_route_kernel, dim3(1), dim3(128), 0, s, E, offsets, aux, z_loss);
}

}  // namespace topmoe
