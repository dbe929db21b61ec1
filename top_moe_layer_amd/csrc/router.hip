// Router: logits r = W_router x, p = softmax(r), S = TopK(p, k) and the
// renormalised weights alpha = p_S / (sum p_S + 1e-20), one token per
// wavefront (MiniMind lesson 13, section 1.5 router equations and walkthrough
// steps 4-5).  Each block also emits, for its tokens, the per-expert
// selection counts and the per-expert sums of p that the offsets and
// load-balancing loss need (lesson 13, section 1.6).
//
// Layout of the work: lane l owns x[h] for h = 4l + 256i; for every expert it
// accumulates a partial dot product with W_router (E partials per lane).  A
// transposing butterfly then leaves expert e's full logit on lane e with
// E - 1 + log2(64/E) shuffles instead of E * 6.
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

template <typename T, int EP>
__global__ __launch_bounds__(256) void router_kernel(
    const T* __restrict__ x, const float* __restrict__ Wr, int64_t N, int H, int E, int k,
    int tb, int32_t* __restrict__ topk_idx, float* __restrict__ alpha,
    int32_t* __restrict__ count_part, float* __restrict__ psum_part) {
  constexpr int LOG_EP = Log2<EP>::v;
  __shared__ int s_cnt[64];
  __shared__ float s_ps[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) s_cnt[tid] = 0;
  __syncthreads();

  const int64_t t0 = int64_t(blockIdx.x) * tb;
  const int64_t t1 = min(N, t0 + tb);
  float psum = 0.f;  // lane e: sum over this wave's tokens of p_{t,e}

  for (int64_t t = t0 + wave; t < t1; t += 4) {
    float acc[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = 0.f;
    const T* xr = x + t * H;
    for (int h = lane * 4; h < H; h += 256) {
      float xv[4];
      load4<T>(xr + h, xv);
#pragma unroll
      for (int e = 0; e < EP; ++e) {
        if (e < E) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(Wr + int64_t(e) * H + h);
          float a = acc[e];
          a = fmaf(xv[0], w.x, a);
          a = fmaf(xv[1], w.y, a);
          a = fmaf(xv[2], w.z, a);
          a = fmaf(xv[3], w.w, a);
          acc[e] = a;
        }
      }
    }
    // Transposing butterfly: after step s each lane keeps half of its values,
    // so after log2(EP) steps lane l holds expert l >> (6 - log2 EP).
#pragma unroll
    for (int s = 0; s < LOG_EP; ++s) {
      const int o = 32 >> s;
      const int half = (EP >> s) >> 1;
      const bool upper = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < EP / 2; ++i) {
        if (i < half) {
          const float send = upper ? acc[i] : acc[i + half];
          const float keep = upper ? acc[i + half] : acc[i];
          acc[i] = keep + __shfl_xor(send, o, 64);
        }
      }
    }
#pragma unroll
    for (int o = 32 >> LOG_EP; o > 0; o >>= 1) acc[0] += __shfl_xor(acc[0], o, 64);
    const float r_lane = __shfl(acc[0], (lane << (6 - LOG_EP)) & 63, 64);

    // softmax over the E logits held by lanes 0..E-1
    const float r = lane < E ? r_lane : -INFINITY;
    const float m = wave_max(r);
    const float ex = lane < E ? expf(r - m) : 0.f;
    const float s = wave_sum(ex);
    const float p = ex / s;
    psum += p;

    // top-k: k rounds of a wave-wide max over (p bits, 64 - lane); larger p
    // first, equal p to the lower expert id.  p >= 0, so its bits order it.
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

  s_ps[wave][lane] = psum;
  __syncthreads();
  if (tid < E) {
    const int64_t o = int64_t(blockIdx.x) * E + tid;
    psum_part[o] = (s_ps[0][tid] + s_ps[1][tid]) + (s_ps[2][tid] + s_ps[3][tid]);
    count_part[o] = s_cnt[tid];
  }
}

template <typename T>
hipError_t launch_router_t(const T* x, const float* Wr, int64_t N, int H, int E, int k, int tb,
                           int nblk, int32_t* topk_idx, float* alpha, int32_t* count_part,
                           float* psum_part, hipStream_t s) {
#define TOPMOE_ROUTER(EPV)                                                                  \
  hipLaunchKernelGGL((router_kernel<T, EPV>), dim3(nblk), dim3(256), 0, s, x, Wr, N, H, E, \
                     k, tb, topk_idx, alpha, count_part, psum_part)
  if (E <= 1) TOPMOE_ROUTER(1);
  else if (E <= 2) TOPMOE_ROUTER(2);
  else if (E <= 4) TOPMOE_ROUTER(4);
  else if (E <= 8) TOPMOE_ROUTER(8);
  else if (E <= 16) TOPMOE_ROUTER(16);
  else if (E <= 32) TOPMOE_ROUTER(32);
  else TOPMOE_ROUTER(64);
#undef TOPMOE_ROUTER
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const void* x, const float* Wr, int dtype, int64_t N, int H, int E,
                         int k, int tb, int nblk, int32_t* topk_idx, float* alpha,
                         int32_t* count_part, float* psum_part, hipStream_t s) {
  if (nblk <= 0) return hipSuccess;
  if (dtype == TOPMOE_DTYPE_FP32)
    return launch_router_t(static_cast<const float*>(x), Wr, N, H, E, k, tb, nblk, topk_idx,
                           alpha, count_part, psum_part, s);
  return launch_router_t(static_cast<const bf16_t*>(x), Wr, N, H, E, k, tb, nblk, topk_idx,
                         alpha, count_part, psum_part, s);
}

}  // namespace topmoe
