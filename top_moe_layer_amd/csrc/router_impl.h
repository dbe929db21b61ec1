// Router building blocks shared by the router kernels and by the decode
// gate/up launch, whose extra blocks route while the GEMM blocks stream
// weights.  Logits r = W_router x, p = softmax(r), S = TopK(p, k) and the
// weights alpha = p_S / (sum p_S + 1e-20), or p_S as it is when the config's
// norm_topk_prob is off (MiniMind lesson 13, section 1.5 router equations and
// walkthrough steps 4-5); per router block, the per-expert selection counts
// and sums of p (lesson 13, section 1.6) and the sum of logsumexp(r)^2 (the
// router z-loss).
#pragma once

#include "device_common.h"

namespace topmoe {
namespace rt {

template <int EP>
struct Log2 { static constexpr int v = 1 + Log2<EP / 2>::v; };
template <>
struct Log2<1> { static constexpr int v = 0; };

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

// Reductions over lanes 0..W-1 (and, identically, every aligned group of W).
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <int W>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// Softmax over the E logits of each of TPW tokens (token u's logit e on lane
// e < E of r[u]), then k rounds of a max over (p bits, 64 - lane): larger p
// first, equal p to the lower expert id (p >= 0, so its bits order it).  The
// TPW tokens go through each step together, so their shuffle chains overlap.
// Writes topk_idx / alpha of the valid tokens, counts their selections in
// s_cnt and adds their p to psum (lane e).
template <int EP, int TPW>
__device__ __forceinline__ void route_tokens(const float (&r)[TPW], int lane, int E, int k,
                                             bool renorm, int64_t t_first, int64_t t_end,
                                             int32_t* __restrict__ topk_idx,
                                             float* __restrict__ alpha,
                                             float* __restrict__ probs,
                                             float* __restrict__ lse_out, int* s_cnt,
                                             float& psum, float& zsum) {
  const bool expert_lane = lane < E;
  float p[TPW];
  uint64_t key[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const float ru = expert_lane ? r[u] : -INFINITY;
    const float m = group_max<EP>(ru);
    const float ex = expert_lane ? expf(ru - m) : 0.f;
    const float sum = group_sum<EP>(ex);
    if (lane == 0 && t_first + u < t_end) {  // z-loss term: logsumexp of the logits, squared
      const float lse = m + logf(sum);
      zsum += lse * lse;
      if (lse_out != nullptr) lse_out[t_first + u] = lse;
    }
    p[u] = expert_lane ? ex / sum : 0.f;  // (lanes past EP see an all-zero group)
    if (t_first + u < t_end) {
      psum += p[u];
      if (probs != nullptr && expert_lane) probs[(t_first + u) * E + lane] = p[u];
    }
    key[u] = expert_lane ? ((uint64_t(__float_as_uint(p[u])) << 32) | uint32_t(64 - lane)) : 0ull;
  }
  int my_e[TPW];
  float my_p[TPW], ssum[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) { my_e[u] = 0; my_p[u] = 0.f; ssum[u] = 0.f; }
  for (int j = 0; j < k; ++j) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const uint64_t best = group_max_u64<EP>(key[u]);
      const int e = 64 - int(uint32_t(best));
      const float pv = __uint_as_float(uint32_t(best >> 32));
      ssum[u] += pv;
      if (lane == j) { my_e[u] = e; my_p[u] = pv; }
      if (lane == e) key[u] = 0ull;
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int64_t t = t_first + u;
    if (lane < k && t < t_end) {
      topk_idx[t * k + lane] = my_e[u];
      alpha[t * k + lane] = renorm ? my_p[u] / (ssum[u] + 1e-20f) : my_p[u];
      atomicAdd(&s_cnt[my_e[u]], 1);  // integer count: order-independent
    }
  }
}

// Block epilogue: per-expert count and sum of p of router block `blk`'s
// tokens, written expert-major at [e * nblk + blk].
__device__ __forceinline__ void write_block_partials(int tid, int E, int nblk, int blk,
                                                     const int* s_cnt, const float (*s_ps)[64],
                                                     int32_t* __restrict__ count_part,
                                                     float* __restrict__ psum_part) {
  if (tid < E) {
    const int64_t o = int64_t(tid) * nblk + blk;
    psum_part[o] = (s_ps[0][tid] + s_ps[1][tid]) + (s_ps[2][tid] + s_ps[3][tid]);
    count_part[o] = s_cnt[tid];
  }
}

// Split layout (large W_router, or few tokens): router block `blk` routes its
// tokens [blk * tb, blk * tb + tb) one at a time, the first four wavefronts of
// the workgroup splitting H into quarters (the wavefronts of a larger
// workgroup beyond those only take part in the barriers, so the arithmetic,
// and the result, is that of a four-wavefront block).  Partial logits meet in
// LDS (s_part) and wavefront 0 finishes the token.  Each wavefront issues the
// loads of CG groups of 256 elements (its x and the matching W_router columns
// of up to 16 experts) before their arithmetic.  Experts past E read row E-1
// (in bounds); their lanes are masked later.  Every thread of the workgroup
// must call it.
template <typename T, int EP>
__device__ __forceinline__ void route_split_block(
    const T* __restrict__ x, const float* __restrict__ Wr, int64_t N, int H, int E, int k,
    bool renorm, int tb, int blk, int nblk, int32_t* __restrict__ topk_idx,
    float* __restrict__ alpha, float* __restrict__ probs, float* __restrict__ lse_out,
    int32_t* __restrict__ count_part, float* __restrict__ psum_part, float* __restrict__ z_part,
    int* s_cnt, float (*s_part)[64], float (*s_ps)[64]) {
  constexpr int CG = EP <= 16 ? 2 : 1;   // groups of 256 elements in flight per wavefront
  constexpr int EC = EP < 16 ? EP : 16;  // experts' W_router columns held at once
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool active = wave < 4;
  if (tid < 64) s_cnt[tid] = 0;
  const int hq = H >> 2;  // H is a multiple of 64, so hq is a multiple of 16
  const int hbeg = wave * hq, hend = hbeg + hq;
  const int64_t t0 = int64_t(blk) * tb;
  const int64_t t1 = (t0 + tb < N) ? t0 + tb : N;
  const f32x4* W4 = reinterpret_cast<const f32x4*>(Wr);
  const int h4 = H >> 2;
  float psum = 0.f;
  float zsum = 0.f;  // thread 0: sum of logsumexp^2 over the block's tokens
  for (int64_t t = t0; t < t1; ++t) {
    float rq = 0.f;
    if (active) {
      float acc[EP];
#pragma unroll
      for (int e = 0; e < EP; ++e) acc[e] = 0.f;
      const T* xr = x + t * H;
      for (int hh = hbeg; hh < hend; hh += 256 * CG) {  // wave-uniform trip count
        float xv[CG][4];
        int q[CG];
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          const int h = hh + 256 * c + lane * 4;
          const bool ok = h < hend;
          q[c] = (ok ? h : hbeg) >> 2;
          load4<T>(xr + 4 * q[c], xv[c]);
          if (!ok) xv[c][0] = xv[c][1] = xv[c][2] = xv[c][3] = 0.f;
        }
#pragma unroll
        for (int e0 = 0; e0 < EP; e0 += EC) {  // W_router columns of EC experts at a time
          f32x4 w[CG][EC];
#pragma unroll
          for (int c = 0; c < CG; ++c)
#pragma unroll
            for (int e = 0; e < EC; ++e)
              w[c][e] = W4[int64_t(e0 + e < E ? e0 + e : E - 1) * h4 + q[c]];
#pragma unroll
          for (int c = 0; c < CG; ++c)
#pragma unroll
            for (int e = 0; e < EC; ++e) {
              float a = acc[e0 + e];
              a = fmaf(xv[c][0], w[c][e].x, a);
              a = fmaf(xv[c][1], w[c][e].y, a);
              a = fmaf(xv[c][2], w[c][e].z, a);
              a = fmaf(xv[c][3], w[c][e].w, a);
              acc[e0 + e] = a;
            }
        }
      }
      rq = reduce_logits<EP>(acc, lane);
    }
    __syncthreads();  // previous token's s_part reads are done
    if (active && lane < E) s_part[wave][lane] = rq;
    __syncthreads();
    if (wave == 0) {
      const float r[1] = {(s_part[0][lane] + s_part[1][lane]) + (s_part[2][lane] + s_part[3][lane])};
      route_tokens<EP, 1>(r, lane, E, k, renorm, t, t1, topk_idx, alpha, probs, lse_out, s_cnt,
                          psum, zsum);
    }
  }
  if (active) s_ps[wave][lane] = psum;  // only wave 0 routed: the other rows are zero
  __syncthreads();
  write_block_partials(tid, E, nblk, blk, s_cnt, s_ps, count_part, psum_part);
  if (tid == 0) z_part[blk] = zsum;
}

// route_split_block for any E <= 16, with the power of two EP >= E that the
// split router kernel uses for that E (the same arithmetic, the same bits).
template <typename T>
__device__ __forceinline__ void route_split_block_upto16(
    const T* __restrict__ x, const float* __restrict__ Wr, int64_t N, int H, int E, int k,
    bool renorm, int tb, int blk, int nblk, int32_t* __restrict__ topk_idx,
    float* __restrict__ alpha, int32_t* __restrict__ count_part, float* __restrict__ psum_part,
    float* __restrict__ z_part, int* s_cnt, float (*s_part)[64], float (*s_ps)[64]) {
#define TOPMOE_RSB(EPV)                                                                        \
  route_split_block<T, EPV>(x, Wr, N, H, E, k, renorm, tb, blk, nblk, topk_idx, alpha, nullptr, \
                            nullptr, count_part, psum_part, z_part, s_cnt, s_part, s_ps)
  if (E <= 1) TOPMOE_RSB(1);
  else if (E <= 2) TOPMOE_RSB(2);
  else if (E <= 4) TOPMOE_RSB(4);
  else if (E <= 8) TOPMOE_RSB(8);
  else TOPMOE_RSB(16);
#undef TOPMOE_RSB
}

}  // namespace rt
}  // namespace topmoe
