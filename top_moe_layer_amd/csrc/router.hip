// Router: logits r = W_router x, p = softmax(r), S = TopK(p, k) and the
// weights alpha = p_S / (sum p_S + 1e-20), or p_S as it is when the config's
// norm_topk_prob is off (MiniMind lesson 13,
// section 1.5 router equations and walkthrough steps 4-5).  Each block also
// emits, for its tokens, the per-expert selection counts and the per-expert
// sums of p that the offsets and load-balancing loss need (lesson 13, section
// 1.6), stored expert-major ([E, blocks]) so the offset scan reads them
// contiguously, and the sum over its tokens of logsumexp(r)^2 for the router
// z-loss (named in the study notes' section 10 table; the squared
// logsumexp is the standard form, a reading).
//
// Work layout: a lane owns x[h] for h = 4l + 256g (of the whole row or of one
// quarter of it) and accumulates one partial dot product per expert; a
// transposing butterfly then leaves expert e's logit on lane e.  Softmax and
// top-k reduce over the first EP lanes only (EP = E rounded up to a power of
// two; the other lanes hold -inf / 0 and would not change the result).
#include "device_common.h"
#include "kernels.h"
#include "router_impl.h"

#include "../../include/topmoe.h"

namespace topmoe {

namespace {

using namespace rt;

// Sum over the 4 lanes of a quad (lanes 4q..4q+3) with two DPP moves; every
// lane of the quad gets (v0 + v1) + (v2 + v3) (the same bits, as + commutes).
__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // xor 1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // xor 2
  return v;
}

// Sum over each group of P (4 or 16) consecutive lanes, the same value in
// every lane of the group: the quad sum, then the two quads of each half row
// (half-row mirror: lane i with 7 - i), then the two halves of the row (row
// mirror: lane i with 15 - i).
template <int P>
__device__ __forceinline__ float lane_group_sum(float v) {
  v = quad_sum(v);
  if constexpr (P == 16) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  }
  return v;
}

template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& q, float (&v)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4& q, float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(q[i]);
}
template <>
__device__ __forceinline__ void unpack16<bf16_t>(const u32x4& q, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(q[i] << 16);
    v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
  }
}

// Mode LDS (EP * H * 4 <= 64 KB): a block routes 16 tokens per pass with P
// lanes per token: P = 4 (one wavefront), or P = 16 where H is a multiple of
// 16 loads (four wavefronts, four tokens each: four times the lanes for the
// same tokens).  W_router is copied into LDS once per block with
// direct-to-LDS loads (all in flight together) and padded with zero rows to
// EP experts.  Lane P u + j of token u loads 16-byte pieces j, j + P, j + 2P,
// ... of the token's row (the token's lanes read 16 P contiguous bytes per
// load) and accumulates E partial logits against W_router columns read from
// LDS; a sum over the P lanes completes the logits, and every lane of the
// group then runs the softmax and the top-k of its token on its own, with no
// cross-lane traffic.  The block owns tokens [t0, t0 + tb).  Per-expert sums
// of p go through LDS in token order.
template <typename T, int EP, int P>
__global__ __launch_bounds__(16 * P) void router_lds_kernel(
    const T* __restrict__ x, const float* __restrict__ Wr, int64_t N, int H, int E, int k,
    bool renorm, int tb, int32_t* __restrict__ topk_idx, float* __restrict__ alpha,
    float* __restrict__ probs, float* __restrict__ lse_out, int32_t* __restrict__ count_part,
    float* __restrict__ psum_part, float* __restrict__ z_part) {
  constexpr int VE = 16 / int(sizeof(T));  // elements per 16-byte load
  // bf16 with 16 lanes per token: a lane's 8 x elements meet two consecutive
  // 16-byte W_router pieces, so the 16 lanes of a read would stride 32 bytes
  // (two-way LDS bank conflicts).  The copy into LDS then permutes each block
  // of 32 pieces so that piece j of every lane's pair lies in one run of 16.
  constexpr bool WPERM = P == 16 && VE == 8;
  constexpr int CI = 8;                    // loads per lane in flight per chunk
  extern __shared__ __attribute__((aligned(1024))) f32x4 s_w4[];  // [EP, H / 4], 1 KB-rounded
  __shared__ int s_cnt[64];
  __shared__ float s_pt[16][EP + 1];  // p of the pass's 16 tokens
  __shared__ float s_z[16];           // their logsumexp^2 (z-loss)
  constexpr int NT = 16 * P;  // threads: 16 tokens per pass
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = tid % P, tok = tid / P;
  const int h4 = H >> 2;
  const int ni = H / (P * VE);  // loads per lane per row (H is a multiple of P * VE)
  const int64_t t0 = int64_t(blockIdx.x) * tb;
  const int64_t t1 = (t0 + tb < N) ? t0 + tb : N;

  // W_router: 1 KB direct-to-LDS loads (lanes past the real rows fetch a
  // clamped element; those slots are zeroed afterwards).
  const int nreal = E * h4, nall = EP * h4;
  {
    const f32x4* W4 = reinterpret_cast<const f32x4*>(Wr);
    for (int c = wave; c * 64 < nreal; c += NT / 64) {
      int i = c * 64 + lane;
      if constexpr (WPERM) {  // slot 16 j + p of each 32-slot block holds piece 2 p + j
        const int r = lane & 31;
        i = c * 64 + (lane & 32) + 2 * (r & 15) + (r >> 4);
      }
      __builtin_amdgcn_global_load_lds(W4 + (i < nreal ? i : nreal - 1),
                                       (__attribute__((address_space(3))) void*)(s_w4 + c * 64),
                                       16, 0, 0);
    }
  }
  if (tid < 64) s_cnt[tid] = 0;
  float psum = 0.f;  // thread e < E: sum of p_e over the block's tokens
  float zsum = 0.f;  // thread 0: sum of logsumexp^2 over the block's tokens
  bool staged = false;

  for (int64_t tp = t0; tp < t1; tp += 16) {
    const int64_t t = tp + tok;
    const bool valid = t < t1;
    const T* xr = x + (valid ? t : t1 - 1) * H + part * VE;
    float acc[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = 0.f;
    // Row pieces in chunks of CI loads, double-buffered: chunk c + 1 is in
    // flight while chunk c is multiplied.
    auto load_chunk = [&](int i0, u32x4(&xq)[CI]) {
#pragma unroll
      for (int c = 0; c < CI; ++c) {
        const int i = i0 + c < ni ? i0 + c : ni - 1;
        xq[c] = *reinterpret_cast<const u32x4*>(xr + i * P * VE);
      }
    };
    auto fma_chunk = [&](int i0, const u32x4(&xq)[CI]) {
#pragma unroll
      for (int c = 0; c < CI; ++c) {
        if (i0 + c < ni) {  // wave-uniform
          float xv[VE];
          unpack16<T>(xq[c], xv);
          const int q = (i0 + c) * (P * VE / 4) + part * (VE / 4);  // f32x4 column of xv[0]
          const int qb = (i0 + c) * (P * VE / 4) + part;  // permuted: slot of piece j is qb + 16 j
#pragma unroll
          for (int e = 0; e < EP; ++e) {
#pragma unroll
            for (int j = 0; j < VE / 4; ++j) {
              const f32x4 w = s_w4[e * h4 + (WPERM ? qb + 16 * j : q + j)];
              float a = acc[e];
              a = fmaf(xv[4 * j + 0], w.x, a);
              a = fmaf(xv[4 * j + 1], w.y, a);
              a = fmaf(xv[4 * j + 2], w.z, a);
              a = fmaf(xv[4 * j + 3], w.w, a);
              acc[e] = a;
            }
          }
        }
      }
    };
    u32x4 xa[CI], xb[CI];
    load_chunk(0, xa);
    if (CI < ni) load_chunk(CI, xb);
    if (!staged) {  // the first row loads are in flight: finish the W_router copy
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
      for (int i = nreal + tid; i < ((nall + 63) & ~63); i += NT)
        s_w4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      staged = true;
    }
    for (int i0 = 0; i0 < ni; i0 += 2 * CI) {
      fma_chunk(i0, xa);
      if (i0 + 2 * CI < ni) load_chunk(i0 + 2 * CI, xa);
      if (i0 + CI < ni) fma_chunk(i0 + CI, xb);
      if (i0 + 3 * CI < ni) load_chunk(i0 + 3 * CI, xb);
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = lane_group_sum<P>(acc[e]);

    // softmax over the E logits (fixed order), in the lane
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < EP; ++e)
      if (e < E) m = fmaxf(m, acc[e]);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      acc[e] = e < E ? expf(acc[e] - m) : 0.f;
      s += acc[e];
    }
    if (part == 0) {  // z-loss term: logsumexp of the logits, squared
      const float lse = m + logf(s);
      s_z[tok] = valid ? lse * lse : 0.f;
      if (lse_out != nullptr && valid) lse_out[t] = lse;
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) acc[e] = acc[e] / s;  // p (0 past E)

    // top-k: k rounds of the largest remaining p, equal p to the lower id;
    // the first sweep gives the renormaliser, the second writes (lane j of
    // the quad writes selections j, j + 4, ...).
    float ssum = 0.f;
    uint64_t taken = 0ull;
    for (int r = 0; renorm && r < k; ++r) {
      int be = 0;
      float bp = -1.f;
#pragma unroll
      for (int e = 0; e < EP; ++e)
        if (e < E && !((taken >> e) & 1ull) && acc[e] > bp) { bp = acc[e]; be = e; }
      taken |= 1ull << be;
      ssum += bp;
    }
    taken = 0ull;
    for (int r = 0; r < k; ++r) {
      int be = 0;
      float bp = -1.f;
#pragma unroll
      for (int e = 0; e < EP; ++e)
        if (e < E && !((taken >> e) & 1ull) && acc[e] > bp) { bp = acc[e]; be = e; }
      taken |= 1ull << be;
      if (valid && r % P == part) {
        topk_idx[t * k + r] = be;
        alpha[t * k + r] = renorm ? bp / (ssum + 1e-20f) : bp;
        atomicAdd(&s_cnt[be], 1);  // integer count: order-independent
      }
    }

    if (part == 0) {
#pragma unroll
      for (int e = 0; e < EP; ++e) s_pt[tok][e] = valid ? acc[e] : 0.f;
    }
    if (probs != nullptr && valid) {  // the softmax for the backward pass (lane part: e = part mod P)
#pragma unroll
      for (int e = 0; e < EP; ++e)
        if (e < E && e % P == part) probs[t * E + e] = acc[e];
    }
    __syncthreads();
    if (tid < E) {
      for (int u = 0; u < 16; ++u) psum += s_pt[u][tid];
    }
    if (tid == 0) {
      for (int u = 0; u < 16; ++u) zsum += s_z[u];
    }
    __syncthreads();
  }

  if (tid < E) {
    const int64_t o = int64_t(tid) * gridDim.x + blockIdx.x;
    psum_part[o] = psum;
    count_part[o] = s_cnt[tid];
  }
  if (tid == 0) z_part[blockIdx.x] = zsum;
}

// Mode split (large W_router, or few tokens): one token at a time per
// four-wavefront block (route_split_block).
template <typename T, int EP>
__global__ __launch_bounds__(256) void router_split_kernel(
    const T* __restrict__ x, const float* __restrict__ Wr, int64_t N, int H, int E, int k,
    bool renorm, int tb, int32_t* __restrict__ topk_idx, float* __restrict__ alpha,
    float* __restrict__ probs, float* __restrict__ lse_out, int32_t* __restrict__ count_part,
    float* __restrict__ psum_part, float* __restrict__ z_part) {
  __shared__ int s_cnt[64];
  __shared__ float s_part[4][64];
  __shared__ float s_ps[4][64];
  route_split_block<T, EP>(x, Wr, N, H, E, k, renorm, tb, int(blockIdx.x), int(gridDim.x),
                           topk_idx, alpha, probs, lse_out, count_part, psum_part, z_part, s_cnt,
                           s_part, s_ps);
}

template <typename T, int EP>
hipError_t launch_router_ep(const T* x, const float* Wr, int64_t N, int H, int E, int k,
                            bool renorm, int tb, int nblk, int mode, int32_t* topk_idx,
                            float* alpha, float* probs, float* lse_out,
                            int32_t* count_part, float* psum_part, float* z_part,
                            const Launch& s) {
  if (mode == ROUTER_MODE_SPLIT)
    return launch_kernel(router_split_kernel<T, EP>, dim3(nblk), dim3(256), 0, s, x, Wr, N, H,
                         E, k, renorm, tb, topk_idx, alpha, probs, lse_out, count_part, psum_part,
                         z_part);
  // W_router rounded up to whole 1 KB direct-to-LDS loads
  const unsigned lds = (unsigned(EP) * unsigned(H) * sizeof(float) + 1023u) & ~1023u;
  if (mode == ROUTER_MODE_LDS16)
    return launch_kernel(router_lds_kernel<T, EP, 16>, dim3(nblk), dim3(256), lds, s, x, Wr, N, H,
                         E, k, renorm, tb, topk_idx, alpha, probs, lse_out, count_part,
                         psum_part, z_part);
  return launch_kernel(router_lds_kernel<T, EP, 4>, dim3(nblk), dim3(64), lds, s, x, Wr, N, H, E,
                       k, renorm, tb, topk_idx, alpha, probs, lse_out, count_part, psum_part,
                       z_part);
}

template <typename T>
hipError_t launch_router_t(const T* x, const float* Wr, int64_t N, int H, int E, int k,
                           bool renorm, int tb, int nblk, int mode, int32_t* topk_idx,
                           float* alpha, float* probs, float* lse_out,
                           int32_t* count_part, float* psum_part, float* z_part,
                           const Launch& s) {
#define TOPMOE_ROUTER(EPV)                                                                 \
  return launch_router_ep<T, EPV>(x, Wr, N, H, E, k, renorm, tb, nblk, mode, topk_idx,    \
                                  alpha, probs, lse_out, count_part, psum_part, z_part, s)
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
                         int k, bool renorm, int tb, int nblk, int mode, int32_t* topk_idx,
                         float* alpha, float* probs, float* lse_out,
                         int32_t* count_part, float* psum_part, float* z_part, const Launch& s) {
  if (nblk <= 0) return hipSuccess;
  if (dtype == TOPMOE_DTYPE_FP32)
    return launch_router_t(static_cast<const float*>(x), Wr, N, H, E, k, renorm, tb, nblk, mode,
                           topk_idx, alpha, probs, lse_out, count_part, psum_part, z_part, s);
  return launch_router_t(static_cast<const bf16_t*>(x), Wr, N, H, E, k, renorm, tb, nblk, mode,
                         topk_idx, alpha, probs, lse_out, count_part, psum_part, z_part, s);
}

}  // namespace topmoe
