// Router: logits r = W_router x, p = softmax(r), S = TopK(p, k) and the
// renormalised weights alpha = p_S / (sum p_S + 1e-20), one token per
// wavefront (MiniMind lesson 13, section 1.5 router equations and walkthrough
// steps 4-5).  Each block also emits, for its tokens, the per-expert
// selection counts and the per-expert sums of p that the offsets and
// load-balancing loss need (lesson 13, section 1.6), stored expert-major
// ([E, blocks]) so the offset scan reads them contiguously.
//
// Work layout: a lane owns x[h] for h = 4l + 256i (of the whole row or of one
// quarter of it) and accumulates one partial dot product per expert; a
// transposing butterfly then leaves expert e's logit on lane e.
#include "device_common.h"
#include "kernels.h"

#include "../../include/topmoe.h"

namespace topmoe {

namespace {

template <typename T>
__device__ __forceinline__ void load4(const T* p, float v[4]);

template <>
__device__ __forceinline__ void load4<float>(const float* p, float v[4]) {
  f32x4 q = *reinterpret_cast<const f32x4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}

template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float v[4]) {
  uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}

template <int EP>
struct Log2 { static constexpr int v = 1 + Log2<EP / 2>::v; };
template <>
struct Log2<1> { static constexpr int v = 0; };

// Transposing butterfly: lane l holds EP partial sums (one per expert); after
// log2(EP) exchange steps each lane keeps one expert, l >> (6 - log2 EP), and
// plain butterfly steps finish the sum.  Lane e (< EP) then receives expert e.
// E - 1 + log2(64 / E) + 1 shuffles instead of 6 E.
// One exchange step of the transposing butterfly (S-th of log2 EP): lanes
// with bit (32 >> S) set keep the upper half of their values, the others the
// lower half, each adding its partner's copy.  Indices are compile-time.
template <int EP, int S>
__device__ __forceinline__ void xpose_step(float (&acc)[EP], int lane) {
  constexpr int o = 32 >> S;
  constexpr int half = (EP >> S) >> 1;
  const bool upper = (lane & o) != 0;
#pragma unroll
  for (int i = 0; i < half; ++i) {
    const float send = upper ? acc[i] : acc[i + half];
    const float keep = upper ? acc[i + half] : acc[i];
    acc[i] = keep + __shfl_xor(send, o, 64);
  }
  if constexpr ((EP >> (S + 1)) > 1) xpose_step<EP, S + 1>(acc, lane);
}

// Transposing butterfly: lane l holds EP partial sums (one per expert); after
// log2(EP) exchange steps each lane keeps one expert, l >> (6 - log2 EP), and
// plain butterfly steps finish the sum.  Lane e (< EP) then receives expert e.
// E - 1 + log2(64 / E) + 1 shuffles instead of 6 E.
template <int EP>
__device__ __forceinline__ float reduce_logits(float (&acc)[EP], int lane) {
  constexpr int LOG_EP = Log2<EP>::v;
  if constexpr (EP > 1) xpose_step<EP, 0>(acc, lane);
#pragma unroll
  for (int o = 32 >> LOG_EP; o > 0; o >>= 1) acc[0] += __shfl_xor(acc[0], o, 64);
  return __shfl(acc[0], (lane << (6 - LOG_EP)) & 63, 64);
}

// Softmax over the E logits held by lanes 0..E-1, then k rounds of a
// wave-wide max over (p bits, 64 - lane): larger p first, equal p to the
// lower expert id (p >= 0, so its bits order it).  Writes topk_idx / alpha
// for token t, counts the selections in s_cnt and adds p to psum (lane e).
__device__ __forceinline__ void route_token(float r_lane, int lane, int E, int k, int64_t t,
                                            int32_t* __restrict__ topk_idx,
                                            float* __restrict__ alpha, int* s_cnt,
                                            float& psum) {
  const float r = lane < E ? r_lane : -INFINITY;
  const float m = wave_max(r);
  const float ex = lane < E ? expf(r - m) : 0.f;
  const float s = wave_sum(ex);
  const float p = ex / s;
  psum += p;
  uint64_t key = lane < E ? ((uint64_t(__float_as_uint(p)) << 32) | uint32_t(64 - lane)) : 0ull;
  int my_e = 0;
  float my_p = 0.f, ssum = 0.f;
  for (int j = 0; j < k; ++j) {
    const uint64_t best = wave_max_u64(key);
    const int e = 64 - int(uint32_t(best));
    const float pv = __uint_as_float(uint32_t(best >> 32));
    ssum += pv;
    if (lane == j) { my_e = e; my_p = pv; }
    if (lane == e) key = 0ull;
  }
  if (lane < k) {
    topk_idx[t * k + lane] = my_e;
    alpha[t * k + lane] = my_p / (ssum + 1e-20f);
    atomicAdd(&s_cnt[my_e], 1);  // integer count: order-independent
  }
}

// Mode 1 (EP * H * 4 <= 64 KB, H <= 2048): the block stages W_router in LDS
// once, padded with zero rows to EP experts; each wavefront routes tokens
// t0 + w, t0 + w + 4, ...  Lane l owns x[h] for h = 4l + 256g; lanes past H
// read a clamped address and use x = 0, so the inner loops have no branches.
// The next token's row is loaded into registers while the current one runs.
template <typename T, int EP>
__global__ __launch_bounds__(256, 1) void router_lds_kernel(
    const T* __restrict__ x, const float* __restrict__ Wr, int64_t N, int H, int E, int k,
    int tb, int32_t* __restrict__ topk_idx, float* __restrict__ alpha,
    int32_t* __restrict__ count_part, float* __restrict__ psum_part) {
  constexpr int NG = 8;  // H <= 256 * NG
  extern __shared__ __attribute__((aligned(16))) f32x4 s_w4[];  // [EP, H / 4]
  __shared__ int s_cnt[64];
  __shared__ float s_ps[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) s_cnt[tid] = 0;
  const int h4 = H >> 2;
  const int nreal = E * h4, nall = EP * h4;
  for (int i = tid; i < nall; i += 256)
    s_w4[i] = i < nreal ? reinterpret_cast<const f32x4*>(Wr)[i] : f32x4{0.f, 0.f, 0.f, 0.f};

  const int ng = (H + 255) >> 8;
  const int64_t t0 = int64_t(blockIdx.x) * tb;
  const int64_t t1 = (t0 + tb < N) ? t0 + tb : N;
  auto load_row = [&](int64_t t, float (&dst)[NG][4]) {
    const T* xr = x + t * H;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g < ng) {  // wave-uniform
        const int h = lane * 4 + 256 * g;
        const bool ok = h < H;
        load4<T>(xr + (ok ? h : 0), dst[g]);
        if (!ok) dst[g][0] = dst[g][1] = dst[g][2] = dst[g][3] = 0.f;
      }
    }
  };
  float psum = 0.f;
  auto compute = [&](int64_t t, const float (&xv)[NG][4]) {
    float acc[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g < ng) {  // wave-uniform
        const int h = lane * 4 + 256 * g;
        const int q = (h < H ? h : 0) >> 2;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
          const f32x4 w = s_w4[e * h4 + q];
          float a = acc[e];
          a = fmaf(xv[g][0], w.x, a);
          a = fmaf(xv[g][1], w.y, a);
          a = fmaf(xv[g][2], w.z, a);
          a = fmaf(xv[g][3], w.w, a);
          acc[e] = a;
        }
      }
    }
    const float r = reduce_logits<EP>(acc, lane);
    route_token(r, lane, E, k, t, topk_idx, alpha, s_cnt, psum);
  };
  // two statically named row buffers, so the prefetch stays in registers
  float xa[NG][4], xb[NG][4];
  int64_t t = t0 + wave;
  if (t < t1) load_row(t, xa);
  __syncthreads();  // W_router staged
  for (; t < t1; t += 8) {
    if (t + 4 < t1) load_row(t + 4, xb);
    compute(t, xa);
    if (t + 4 >= t1) break;
    if (t + 8 < t1) load_row(t + 8, xa);
    compute(t + 4, xb);
  }

  s_ps[wave][lane] = psum;
  __syncthreads();
  if (tid < E) {
    const int64_t o = int64_t(tid) * gridDim.x + blockIdx.x;
    psum_part[o] = (s_ps[0][tid] + s_ps[1][tid]) + (s_ps[2][tid] + s_ps[3][tid]);
    count_part[o] = s_cnt[tid];
  }
}

// Mode 2 (large W_router, or few tokens): the four wavefronts of a block
// split H into quarters of one token; partial logits meet in LDS and
// wavefront 0 finishes the token.  The block walks its tokens in order.
// Experts past E read row E-1 (in bounds); their lanes are masked later.
template <typename T, int EP>
__global__ __launch_bounds__(256, 1) void router_split_kernel(
    const T* __restrict__ x, const float* __restrict__ Wr, int64_t N, int H, int E, int k,
    int tb, int32_t* __restrict__ topk_idx, float* __restrict__ alpha,
    int32_t* __restrict__ count_part, float* __restrict__ psum_part) {
  __shared__ int s_cnt[64];
  __shared__ float s_part[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) s_cnt[tid] = 0;
  const int hq = H >> 2;  // H is a multiple of 64, so hq is a multiple of 16
  const int hbeg = wave * hq, hend = hbeg + hq;
  const int64_t t0 = int64_t(blockIdx.x) * tb;
  const int64_t t1 = (t0 + tb < N) ? t0 + tb : N;
  const f32x4* W4 = reinterpret_cast<const f32x4*>(Wr);
  const int h4 = H >> 2;
  float psum = 0.f;
  for (int64_t t = t0; t < t1; ++t) {
    float acc[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = 0.f;
    const T* xr = x + t * H;
    for (int hh = hbeg; hh < hend; hh += 256) {  // wave-uniform trip count
      const int h = hh + lane * 4;
      const bool ok = h < hend;
      float xv[4];
      load4<T>(xr + (ok ? h : hbeg), xv);
      if (!ok) xv[0] = xv[1] = xv[2] = xv[3] = 0.f;
      const int q = (ok ? h : hbeg) >> 2;
#pragma unroll
      for (int e = 0; e < EP; ++e) {
        const int er = e < E ? e : E - 1;
        const f32x4 w = W4[int64_t(er) * h4 + q];
        float a = acc[e];
        a = fmaf(xv[0], w.x, a);
        a = fmaf(xv[1], w.y, a);
        a = fmaf(xv[2], w.z, a);
        a = fmaf(xv[3], w.w, a);
        acc[e] = a;
      }
    }
    const float rq = reduce_logits<EP>(acc, lane);
    __syncthreads();  // previous token's s_part reads are done
    if (lane < E) s_part[wave][lane] = rq;
    __syncthreads();
    if (wave == 0) {
      const float r = (s_part[0][lane] + s_part[1][lane]) + (s_part[2][lane] + s_part[3][lane]);
      route_token(r, lane, E, k, t, topk_idx, alpha, s_cnt, psum);
    }
  }
  __syncthreads();
  if (tid < E) {
    const int64_t o = int64_t(tid) * gridDim.x + blockIdx.x;
    psum_part[o] = psum;  // wave 0's lanes hold the sums
    count_part[o] = s_cnt[tid];
  }
}

template <typename T>
hipError_t launch_router_t(const T* x, const float* Wr, int64_t N, int H, int E, int k, int tb,
                           int nblk, int mode, int32_t* topk_idx, float* alpha,
                           int32_t* count_part, float* psum_part, const Launch& s) {
  int ep = 1;
  while (ep < E) ep *= 2;
  const size_t lds = mode == ROUTER_MODE_LDS ? size_t(ep) * H * sizeof(float) : 0;
#define TOPMOE_ROUTER(EPV)                                                                  \
  return mode == ROUTER_MODE_LDS                                                            \
             ? launch_kernel(router_lds_kernel<T, EPV>, dim3(nblk), dim3(256), unsigned(lds), \
                             s, x, Wr, N, H, E, k, tb, topk_idx, alpha, count_part, psum_part) \
             : launch_kernel(router_split_kernel<T, EPV>, dim3(nblk), dim3(256), 0, s, x, Wr,  \
                             N, H, E, k, tb, topk_idx, alpha, count_part, psum_part)
  if (E <= 1) TOPMOE_ROUTER(1);
  if (E <= 2) TOPMOE_ROUTER(2);
  if (E <= 4) TOPMOE_ROUTER(4);
  if (E <= 8) TOPMOE_ROUTER(8);
  if (E <= 16) TOPMOE_ROUTER(16);
  if (E <= 32) TOPMOE_ROUTER(32);
  TOPMOE_ROUTER(64);
#undef TOPMOE_ROUTER
}

}  // namespace

hipError_t launch_router(const void* x, const float* Wr, int dtype, int64_t N, int H, int E,
                         int k, int tb, int nblk, int mode, int32_t* topk_idx, float* alpha,
                         int32_t* count_part, float* psum_part, const Launch& s) {
  if (nblk <= 0) return hipSuccess;
  if (dtype == TOPMOE_DTYPE_FP32)
    return launch_router_t(static_cast<const float*>(x), Wr, N, H, E, k, tb, nblk, mode,
                           topk_idx, alpha, count_part, psum_part, s);
  return launch_router_t(static_cast<const bf16_t*>(x), Wr, N, H, E, k, tb, nblk, mode, topk_idx,
                         alpha, count_part, psum_part, s);
}

}  // namespace topmoe
