// Memory-bound kernels of the backward pass: operand transposes, the router
// backward, the dx combine and the router-weight gradient.
//
// The backward follows the forward through the selected weights alpha and
// the mean probabilities in aux: the top-k choice and the per-expert counts
// are discrete and pass no gradient, the softmax probabilities do
// (minimind3 chapter 4, section 4.4; MiniMind study notes, section 7 on how
// the router is trained).  Per token t and selected expert e (slot j):
//   d alpha_{t,j} = dy_t . Expert_e(x_t)                (from the GEMM epilogue)
//   alpha = p_S / (sum p_S + 1e-20):  dp_{S_j} = d alpha_j / Z - sum_i d alpha_i p_{S_i} / Z^2
//     (evaluated as (sum_i p_{S_i} (d alpha_j - d alpha_i) + 1e-20 d alpha_j) / Z^2)
//   (alpha = p_S when the weights are not renormalised: dp_{S_j} = d alpha_j)
//   aux = coef E sum_e c_e (sum_t p_{t,e}) / N^2:  dp_{t,e} += daux coef E c_e / N^2
//   softmax:  dr_e = p_e (dp_e - sum_e' p_e' dp_e');  dx_t += W_r^T dr_t;  dW_r += dr_t x_t^T.
//   router z-loss z_coef * mean_t lse_t^2 (upstream dz):  dr_e += z_coef dz 2 lse_t p_e / N
//   (d lse / d r = p); an entry dropped by an expert capacity passes no d alpha.
// Every float reduction runs in a fixed order, so results repeat bit for bit.
#include "device_common.h"
#include "kernels.h"

#include "../../include/topmoe.h"

namespace topmoe {

namespace {

// 16 bytes of the dtype (8 bf16 or 4 fp32 values) <-> fp32.
template <typename T>
struct Pack {
  static constexpr int n = 16 / int(sizeof(T));
};
template <typename T>
__device__ __forceinline__ void ld16(const T* p, float (&v)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void ld16<float>(const float* p, float (&v)[4]) {
  const f32x4 q = *reinterpret_cast<const f32x4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
template <>
__device__ __forceinline__ void ld16<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(q[i] << 16);
    v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
  }
}
template <typename T>
__device__ __forceinline__ void st16(T* p, const float (&v)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void st16<float>(float* p, const float (&v)[4]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void st16<bf16_t>(bf16_t* p, const float (&v)[8]) {
  u32x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    q[i] = uint32_t(f32_to_bf16(v[2 * i])) | (uint32_t(f32_to_bf16(v[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4*>(p) = q;
}

// ---------------------------------------------------------------- transposes
// Tiles of 64 x 64 elements through LDS: 16-byte row-piece loads, 16-byte
// column-piece stores.  The row stride of the LDS tile is 64 + 16 bytes worth
// of elements so that 16-byte writes stay aligned.
// bf16: the column pass reads 2-byte elements of rows 8 apart, which with the
// padded stride alone put four of every eight lane groups on the same banks;
// the 16-byte piece of row r sits at piece index p ^ ((r / 8) % 8) as well.
template <typename T>
struct TileT {
  static constexpr int V = 16 / int(sizeof(T));  // elements per 16 bytes
  static constexpr int LD = 64 + V;              // LDS row stride (elements)
  static constexpr int CPR = 64 / V;             // 16-byte pieces per 64-element row
  static constexpr int PER = 64 * CPR / 256;     // pieces per thread (256 threads)
  __device__ static int sw(int r) { return sizeof(T) == 2 ? (r >> 3) & 7 : 0; }
  // element (r, c) and 16-byte piece (r, p) of the tile
  __device__ static int at(int r, int c) { return r * LD + (((c / V) ^ sw(r)) * V) + c % V; }
  __device__ static int piece(int r, int p) { return r * LD + (p ^ sw(r)) * V; }
};

// out[b][c][col0 + r] = in[b][r][c] for up to three matrices (blockIdx.z),
// each [batch][R][C] with C, R multiples of 64.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeJobs jobs) {
  using TT = TileT<T>;
  __shared__ __attribute__((aligned(16))) T tile[64 * TT::LD];
  // (constant indices: a run-time index into the argument array would copy
  // it to scratch memory)
  const TransposeJob jb = blockIdx.z == 0 ? jobs.job[0] : blockIdx.z == 1 ? jobs.job[1] : jobs.job[2];
  const int tiles_c = jb.C / 64;
  const int tr = int(blockIdx.x) / tiles_c, tc = int(blockIdx.x) - tr * tiles_c;
  if (tr * 64 >= jb.R) return;
  const int b = int(blockIdx.y);
  if (b >= jb.batch) return;
  const T* src = static_cast<const T*>(jb.src) + int64_t(b) * jb.src_bs;
  T* dst = static_cast<T*>(jb.dst) + int64_t(b) * jb.dst_bs;
  const int r0 = tr * 64, c0 = tc * 64;
#pragma unroll
  for (int i = 0; i < TT::PER; ++i) {
    const int id = int(threadIdx.x) + 256 * i;
    const int r = id / TT::CPR, q = id - r * TT::CPR;
    *reinterpret_cast<u32x4*>(&tile[TT::piece(r, q)]) =
        *reinterpret_cast<const u32x4*>(src + int64_t(r0 + r) * jb.C + c0 + q * TT::V);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TT::PER; ++i) {
    const int id = int(threadIdx.x) + 256 * i;
    const int c = id / TT::CPR, q = id - c * TT::CPR;
    float v[TT::V];
#pragma unroll
    for (int w = 0; w < TT::V; ++w) v[w] = to_f32<T>(tile[TT::at(q * TT::V + w, c)]);
    st16<T>(dst + int64_t(c0 + c) * jb.ldo + jb.col0 + r0 + q * TT::V, v);
  }
}

// Padded group columns: group e's rows (offsets[e] .. offsets[e+1]) sit at
// columns poff_e .. poff_e + c_e of a [C][ldo] matrix, poff_e = sum over
// earlier groups of c rounded up to 64, and columns c_e .. round64(c_e) are
// zero.  out[c][poff_e + i] = scale_g * in[row_g][c] with g = offsets[e] + i,
// row_g = entries[g] / k (entries NULL: g), scale_g = alpha_g[g] (NULL: 1).
// Up to two sources (blockIdx.z) share the grouping.  Grid: x = 64-column
// blocks of the padded width bound, y = C / 64.
template <typename T>
__global__ __launch_bounds__(256) void gather_transpose_kernel(GatherTransposeJobs jobs) {
  using TT = TileT<T>;
  __shared__ __attribute__((aligned(16))) T tile[64 * TT::LD];
  __shared__ int s_grp[4];  // group, its first row, its row count, its first padded column
  const int tid = int(threadIdx.x), lane = tid & 63;
  const int64_t pc0 = int64_t(blockIdx.x) * 64;
  if (tid < 64) {
    const int G = jobs.offsets != nullptr ? jobs.E : 1;
    int c = 0, o0 = 0;
    if (lane < G) {
      o0 = jobs.offsets != nullptr ? jobs.offsets[lane] : 0;
      c = (jobs.offsets != nullptr ? jobs.offsets[lane + 1] : int(jobs.rows)) - o0;
    }
    const int kp = (c + 63) & ~63;
    const int incl = wave_inclusive_scan(kp, lane);
    if (lane == 0) s_grp[0] = -1;
    __builtin_amdgcn_wave_barrier();
    if (lane < G && pc0 >= incl - kp && pc0 < incl) {  // at most one group holds the block
      s_grp[0] = lane;
      s_grp[1] = o0;
      s_grp[2] = c;
      s_grp[3] = incl - kp;
    }
  }
  __syncthreads();
  if (s_grp[0] < 0) return;  // past the last group's padded columns
  const int gfirst = s_grp[1], cnt = s_grp[2], poff = s_grp[3];
  const int local0 = int(pc0) - poff;
  const int h0 = int(blockIdx.y) * 64;
  const GatherTransposeJob jb = blockIdx.z == 0 ? jobs.job[0] : jobs.job[1];
  const T* src = static_cast<const T*>(jb.src);
#pragma unroll
  for (int i = 0; i < TT::PER; ++i) {
    const int id = tid + 256 * i;
    const int l = id / TT::CPR, q = id - l * TT::CPR;
    const int li = local0 + l;
    float v[TT::V];
    if (li < cnt) {
      const int g = gfirst + li;
      const int64_t row = jobs.entries != nullptr ? jobs.entries[g] / jobs.k : g;
      ld16<T>(src + row * jobs.C + h0 + q * TT::V, v);
      if (jb.scale != nullptr) {
        const float s = jb.scale[g];
#pragma unroll
        for (int w = 0; w < TT::V; ++w) v[w] *= s;
      }
    } else {
#pragma unroll
      for (int w = 0; w < TT::V; ++w) v[w] = 0.f;
    }
    st16<T>(&tile[TT::piece(l, q)], v);
  }
  __syncthreads();
  T* dst = static_cast<T*>(jb.dst);
#pragma unroll
  for (int i = 0; i < TT::PER; ++i) {
    const int id = tid + 256 * i;
    const int h = id / TT::CPR, q = id - h * TT::CPR;
    float v[TT::V];
#pragma unroll
    for (int w = 0; w < TT::V; ++w) v[w] = to_f32<T>(tile[TT::at(q * TT::V + w, h)]);
    st16<T>(dst + int64_t(h0 + h) * jobs.ldo + pc0 + q * TT::V, v);
  }
}

// ------------------------------------------------------------ router backward
// EP lanes per token (lane e: expert e), 64 / EP tokens per wavefront.
template <int EP>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = EP / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int EP>
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const float* __restrict__ probs, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dalpha_part, int nt, const int32_t* __restrict__ counts_off,
    const uint8_t* __restrict__ keep, const float* __restrict__ lse, int64_t N, int E, int k,
    bool renorm, float aux_scale, const float* __restrict__ aux_mul, float z_scale,
    const float* __restrict__ z_mul, float* __restrict__ dr) {
  constexpr int TPW = 64 / EP;
  const int lane = int(threadIdx.x) & 63, wave = int(threadIdx.x) >> 6;
  const int u = lane / EP, e = lane - u * EP, base = u * EP;
  const int64_t t = (int64_t(blockIdx.x) * 4 + wave) * TPW + u;
  const bool valid = t < N;
  const bool el = valid && e < E;
  const float p = el ? probs[t * E + e] : 0.f;
  // lane j < k of the group: slot j's expert, d alpha (sum of the column-tile
  // partials in order) and selected probability
  int ej = 0;
  float dal = 0.f;
  if (valid && e < k) {
    ej = topk_idx[t * k + e];
    if (keep == nullptr || keep[t * k + e] != 0) {  // a dropped entry's output was not used
      const float* dp = dalpha_part + (t * k + e) * int64_t(nt);
      for (int c = 0; c < nt; ++c) dal += dp[c];
    }
  }
  const float pj = __shfl(p, base + ej, 64);
  const bool slot = valid && e < k;
  const float z = group_sum<EP>(slot ? pj : 0.f) + 1e-20f;
  // d alpha_j / Z - sum_i d alpha_i p_i / Z^2 = (sum_i p_i (d alpha_j - d alpha_i)
  // + 1e-20 d alpha_j) / Z^2, summed term by term: the plain form cancels
  // (for k = 1 the exact value is 1e-20 d alpha / Z^2).
  float num = 0.f;
  for (int i = 0; i < k; ++i) {
    const float pi = __shfl(pj, base + i, 64);
    const float di = __shfl(dal, base + i, 64);
    num = fmaf(pi, dal - di, num);
  }
  const float dps = renorm ? (num + 1e-20f * dal) / (z * z) : dal;
  // d p_e: the slot holding e (if any), plus the aux term
  float dp = 0.f;
  for (int j = 0; j < k; ++j) {
    const int ex = __shfl(ej, base + j, 64);
    const float v = __shfl(dps, base + j, 64);
    if (ex == e) dp = v;
  }
  // the loss terms' upstream gradients: host factors times optional device scalars
  if (aux_mul != nullptr) aux_scale *= aux_mul[0];
  if (z_mul != nullptr) z_scale *= z_mul[0];
  if (el && aux_scale != 0.f) dp += aux_scale * float(counts_off[e + 1] - counts_off[e]);
  const float dot = group_sum<EP>(el ? p * dp : 0.f);
  float g = p * (dp - dot);
  if (lse != nullptr && el) g = fmaf(z_scale * lse[t], p, g);
  if (el) dr[t * E + e] = g;
}

// ------------------------------------------------------------------- combine
// dx[t] = sum of the k slot rows of token t in ascending expert id (each in
// the dtype, like the forward combine) + sum_e dr[t][e] W_r[e], accumulated
// in fp32 and rounded once.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const T* __restrict__ slots, const int32_t* __restrict__ topk_idx,
    const uint8_t* __restrict__ keep, const float* __restrict__ dr,
    const float* __restrict__ Wr, int64_t N, int H, int E, int k, T* __restrict__ dx) {
  constexpr int V = Pack<T>::n;
  const int hv = H / V;
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= N * hv) return;
  const int64_t t = gid / hv;
  const int h = int(gid - t * hv) * V;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  const int32_t* ids = topk_idx + t * k;
  int prev = -1;
  for (int r = 0; r < k; ++r) {
    int best_j = 0, best_e = 1 << 30;
    for (int j = 0; j < k; ++j) {
      const int e = ids[j];
      if (e > prev && e < best_e) { best_e = e; best_j = j; }
    }
    prev = best_e;
    if (keep != nullptr && keep[t * k + best_j] == 0) continue;  // dropped: no expert term
    float v[V];
    ld16<T>(slots + (t * k + best_j) * H + h, v);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += v[i];
  }
  const float* drt = dr + t * E;
  for (int e = 0; e < E; ++e) {
    const float d = drt[e];
    const float* w = Wr + int64_t(e) * H + h;
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(w + i);
      acc[i] = fmaf(d, q.x, acc[i]);
      acc[i + 1] = fmaf(d, q.y, acc[i + 1]);
      acc[i + 2] = fmaf(d, q.z, acc[i + 2]);
      acc[i + 3] = fmaf(d, q.w, acc[i + 3]);
    }
  }
  st16<T>(dx + t * H + h, acc);
}

// ------------------------------------------------------- router weight grad
// dW_r[e][h] = sum_t dr[t][e] x[t][h], split over token chunks of kDwrChunk
// (64: enough blocks to fill the chip at a few thousand tokens): block
// (512-column block, chunk) has four wavefronts of 16 tokens each; a lane
// owns 8 consecutive columns and 8 experts at a time.  The four wavefronts'
// sums meet in LDS in a fixed order and the block writes one partial per
// chunk; a second kernel sums the chunks (again in a fixed order).
constexpr int kDwrWaves = 4;
constexpr int kDwrTpw = kDwrChunk / kDwrWaves;  // tokens per wavefront
static_assert(kDwrTpw % 4 == 0, "whole groups of four rows per wavefront");

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    ld16<T>(p, v);
  } else {
    float a[4], b[4];
    ld16<T>(p, a);
    ld16<T>(p + 4, b);
#pragma unroll
    for (int w = 0; w < 4; ++w) { v[w] = a[w]; v[w + 4] = b[w]; }
  }
}

// A lane's 8 partial sums of one expert row in LDS: two 16-byte halves, each
// in a 1 KB run of the 64 lanes' halves (16-byte accesses of consecutive
// lanes, no bank conflicts; lane * 8 + b strode 32 bytes).
__device__ __forceinline__ int dwr_slot(int lane, int b) {
  return (b >> 2) * 256 + lane * 4 + (b & 3);
}

template <typename T>
__global__ __launch_bounds__(256) void dwr_partial_kernel(const T* __restrict__ x,
                                                          const float* __restrict__ dr,
                                                          int64_t N, int H, int E,
                                                          float* __restrict__ part) {
  __shared__ float s_dr[kDwrChunk * 8];                 // this expert chunk's dr rows
  __shared__ float s_acc[kDwrWaves - 1][8][8 * 64 + 4];  // waves 1..3: 8 experts x 512 columns
  const int tid = int(threadIdx.x), lane = tid & 63, wave = tid >> 6;
  const int h = int(blockIdx.x) * 512 + lane * 8;
  const bool hok = h < H;
  const int64_t t0 = int64_t(blockIdx.y) * kDwrChunk;
  const int nt = int(N - t0 < kDwrChunk ? N - t0 : kDwrChunk);
  const int tw0 = wave * kDwrTpw;  // this wave's tokens in the chunk
  const int ntw = nt - tw0 < 0 ? 0 : (nt - tw0 < kDwrTpw ? nt - tw0 : kDwrTpw);
  for (int e0 = 0; e0 < E; e0 += 8) {
    __syncthreads();  // the previous expert chunk's LDS reads are done
    for (int i = tid; i < kDwrChunk * 8; i += 256) {
      const int t = i >> 3, e = e0 + (i & 7);
      s_dr[i] = (t < nt && e < E) ? dr[(t0 + t) * E + e] : 0.f;
    }
    __syncthreads();
    float acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[a][b] = 0.f;
    if (hok) {
      int i = 0;
      for (; i + 4 <= ntw; i += 4) {  // four rows in flight
        float xv[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) load8<T>(x + (t0 + tw0 + i + r) * H + h, xv[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int a = 0; a < 8; ++a) {
            const float d = s_dr[(tw0 + i + r) * 8 + a];
#pragma unroll
            for (int b = 0; b < 8; ++b) acc[a][b] = fmaf(d, xv[r][b], acc[a][b]);
          }
      }
      for (; i < ntw; ++i) {
        float xv[8];
        load8<T>(x + (t0 + tw0 + i) * H + h, xv);
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          const float d = s_dr[(tw0 + i) * 8 + a];
#pragma unroll
          for (int b = 0; b < 8; ++b) acc[a][b] = fmaf(d, xv[b], acc[a][b]);
        }
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) s_acc[wave - 1][a][dwr_slot(lane, b)] = acc[a][b];
    }
    __syncthreads();
    if (wave == 0 && hok) {
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        if (e0 + a >= E) break;
        float v[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          float sum = acc[a][b];
#pragma unroll
          for (int w = 0; w < kDwrWaves - 1; ++w) sum += s_acc[w][a][dwr_slot(lane, b)];
          v[b] = sum;
        }
        float* o = part + (int64_t(blockIdx.y) * E + e0 + a) * H + h;
        *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
  }
}

// dW_r[i] = sum over chunks c (ascending) of part[c][i]: 64 outputs per block,
// four threads per output take every fourth chunk, then meet in LDS in order.
__global__ __launch_bounds__(256) void dwr_reduce_kernel(const float* __restrict__ part,
                                                         int nchunk, int64_t EH,
                                                         float* __restrict__ dWr) {
  __shared__ float s_sum[4][64];
  const int tid = int(threadIdx.x), o = tid & 63, q = tid >> 6;
  const int64_t i = int64_t(blockIdx.x) * 64 + o;
  float s = 0.f;
  if (i < EH) {
    int c = q;
    for (; c + 12 < nchunk; c += 16) {  // four loads in flight
      const float a = part[int64_t(c) * EH + i], b = part[int64_t(c + 4) * EH + i];
      const float d = part[int64_t(c + 8) * EH + i], e = part[int64_t(c + 12) * EH + i];
      s += a; s += b; s += d; s += e;
    }
    for (; c < nchunk; c += 4) s += part[int64_t(c) * EH + i];
  }
  s_sum[q][o] = s;
  __syncthreads();
  if (q == 0 && i < EH) dWr[i] = (s_sum[0][o] + s_sum[1][o]) + (s_sum[2][o] + s_sum[3][o]);
}

template <int EP>
hipError_t launch_router_bwd_ep(const float* probs, const int32_t* topk_idx,
                                const float* dalpha_part, int nt, const int32_t* counts_off,
                                const uint8_t* keep, const float* lse, int64_t N, int E, int k,
                                bool renorm, float aux_scale, const float* aux_mul,
                                float z_scale, const float* z_mul, float* dr, const Launch& s) {
  constexpr int TPB = 4 * (64 / EP);  // tokens per block
  const int64_t grid = (N + TPB - 1) / TPB;
  return launch_kernel(router_bwd_kernel<EP>, dim3(unsigned(grid)), dim3(256), 0, s, probs,
                       topk_idx, dalpha_part, nt, counts_off, keep, lse, N, E, k, renorm,
                       aux_scale, aux_mul, z_scale, z_mul, dr);
}

}  // namespace

hipError_t launch_transpose(int dtype, const TransposeJobs& jobs, int max_tiles, int max_batch,
                            const Launch& s) {
  if (jobs.n <= 0 || max_tiles <= 0 || max_batch <= 0) return hipSuccess;
  const dim3 grid(unsigned(max_tiles), unsigned(max_batch), unsigned(jobs.n));
  if (dtype == TOPMOE_DTYPE_FP32)
    return launch_kernel(transpose_kernel<float>, grid, dim3(256), 0, s, jobs);
  return launch_kernel(transpose_kernel<bf16_t>, grid, dim3(256), 0, s, jobs);
}

hipError_t launch_gather_transpose(int dtype, const GatherTransposeJobs& jobs, int64_t ldo,
                                   const Launch& s) {
  if (jobs.n <= 0 || ldo <= 0 || jobs.C <= 0) return hipSuccess;
  const dim3 grid(unsigned(ldo / 64), unsigned(jobs.C / 64), unsigned(jobs.n));
  if (dtype == TOPMOE_DTYPE_FP32)
    return launch_kernel(gather_transpose_kernel<float>, grid, dim3(256), 0, s, jobs);
  return launch_kernel(gather_transpose_kernel<bf16_t>, grid, dim3(256), 0, s, jobs);
}

hipError_t launch_router_bwd(const float* probs, const int32_t* topk_idx,
                             const float* dalpha_part, int nt, const int32_t* counts_off,
                             const uint8_t* keep, const float* lse, int64_t N, int E, int k,
                             bool renorm, float aux_scale, const float* aux_mul,
                             float z_scale, const float* z_mul, float* dr, const Launch& s) {
  if (N <= 0) return hipSuccess;
#define TOPMOE_RB(EPV)                                                                       \
  return launch_router_bwd_ep<EPV>(probs, topk_idx, dalpha_part, nt, counts_off, keep, lse, N, \
                                   E, k, renorm, aux_scale, aux_mul, z_scale, z_mul, dr, s)
  if (E <= 1) TOPMOE_RB(1);
  if (E <= 2) TOPMOE_RB(2);
  if (E <= 4) TOPMOE_RB(4);
  if (E <= 8) TOPMOE_RB(8);
  if (E <= 16) TOPMOE_RB(16);
  if (E <= 32) TOPMOE_RB(32);
  TOPMOE_RB(64);
#undef TOPMOE_RB
}

hipError_t launch_combine_bwd(const void* slots, const int32_t* topk_idx, const uint8_t* keep,
                              const float* dr, const float* Wr, int64_t N, int H, int E, int k,
                              int dtype, void* dx, const Launch& s) {
  const int64_t work = N * (H / (dtype == TOPMOE_DTYPE_FP32 ? 4 : 8));
  if (work <= 0) return hipSuccess;
  const int64_t grid = (work + 255) / 256;
  if (dtype == TOPMOE_DTYPE_FP32)
    return launch_kernel(combine_bwd_kernel<float>, dim3(unsigned(grid)), dim3(256), 0, s,
                         static_cast<const float*>(slots), topk_idx, keep, dr, Wr, N, H, E, k,
                         static_cast<float*>(dx));
  return launch_kernel(combine_bwd_kernel<bf16_t>, dim3(unsigned(grid)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(slots), topk_idx, keep, dr, Wr, N, H, E, k,
                       static_cast<bf16_t*>(dx));
}

int dwr_chunks(int64_t N) { return int((N + kDwrChunk - 1) / kDwrChunk); }

hipError_t launch_dwr(const void* x, const float* dr, int64_t N, int H, int E, int dtype,
                      float* part, float* dWr, const Launch& s) {
  const int nchunk = dwr_chunks(N);
  Launch first = s, second = s;
  first.stop = nullptr;
  second.start = nullptr;
  if (nchunk > 0) {
    const dim3 grid(unsigned((H + 511) / 512), unsigned(nchunk));
    const hipError_t err =
        dtype == TOPMOE_DTYPE_FP32
            ? launch_kernel(dwr_partial_kernel<float>, grid, dim3(256), 0, first,
                            static_cast<const float*>(x), dr, N, H, E, part)
            : launch_kernel(dwr_partial_kernel<bf16_t>, grid, dim3(256), 0, first,
                            static_cast<const bf16_t*>(x), dr, N, H, E, part);
    if (err != hipSuccess) return err;
  } else {
    second.start = s.start;
  }
  const int64_t EH = int64_t(E) * H;
  const hipError_t err = launch_kernel(dwr_reduce_kernel, dim3(unsigned((EH + 63) / 64)),
                                       dim3(256), 0, second, part, nchunk, EH, dWr);
  s.launched = true;
  return err;
}

}  // namespace topmoe
