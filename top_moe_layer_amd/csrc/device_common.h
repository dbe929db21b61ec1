// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace topmoe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Four consecutive values in the dtype (8 bytes of bf16, 16 of fp32).
template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4]);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&v)[4]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float (&v)[4]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const uint32_t a = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
  const uint32_t b = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
  *reinterpret_cast<u32x2*>(p) = u32x2{a, b};
}

template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&v)[4]) {
  const f32x4 q = *reinterpret_cast<const f32x4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float (&v)[4]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 q = *reinterpret_cast<const u32x2*>(p);
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}

// 4 x 4 transpose inside each quad of lanes (q = lane & 3) with two DPP
// quad permutations: on entry lane q holds rows 0..3 of column q, on exit
// row q of columns 0..3.  Step m (m = 1, 2) pairs index r (bit m clear) with
// r ^ m and lane q with q ^ m: the lane whose bit m is clear keeps b[r] and
// sends b[r ^ m], its partner keeps b[r ^ m] and sends b[r]; each puts what it
// receives where its sent value was.  An element (row, col) thus moves only
// when its row and column bits differ, flipping both, which after both steps
// puts it at lane row, index col.  Every lane of the quad must execute it.
template <int M, int CTRL>
__device__ __forceinline__ void quad_exchange(float& lo, float& hi, bool upper) {
  const float send = upper ? lo : hi;
  const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), CTRL, 0xF, 0xF, false));
  if (upper) lo = recv;
  else hi = recv;
}
__device__ __forceinline__ void quad_transpose(float (&b)[4], int q) {
  const bool u1 = (q & 1) != 0, u2 = (q & 2) != 0;
  quad_exchange<1, 0xB1>(b[0], b[1], u1);  // lane ^ 1
  quad_exchange<1, 0xB1>(b[2], b[3], u1);
  quad_exchange<2, 0x4E>(b[0], b[2], u2);  // lane ^ 2
  quad_exchange<2, 0x4E>(b[1], b[3], u2);
}

// Two values of the dtype stored together (the (g, u) pairs of the backward):
// one 4-byte word for bf16 (first value in the low half), 8 bytes for fp32.
template <typename T>
__device__ __forceinline__ void store_pair(void* base, int64_t i, float a, float b);
template <>
__device__ __forceinline__ void store_pair<bf16_t>(void* base, int64_t i, float a, float b) {
  static_cast<uint32_t*>(base)[i] = uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16);
}
template <>
__device__ __forceinline__ void store_pair<float>(void* base, int64_t i, float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  static_cast<f32x2*>(base)[i] = f32x2{a, b};
}
// Pairs i .. i+3 (first values a[], second values b[]) in one or two 16-byte stores.
template <typename T>
__device__ __forceinline__ void store_pairs4(void* base, int64_t i, const float (&a)[4],
                                             const float (&b)[4]);
template <>
__device__ __forceinline__ void store_pairs4<bf16_t>(void* base, int64_t i, const float (&a)[4],
                                                     const float (&b)[4]) {
  u32x4 q;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    q[w] = uint32_t(f32_to_bf16(a[w])) | (uint32_t(f32_to_bf16(b[w])) << 16);
  *reinterpret_cast<u32x4*>(static_cast<uint32_t*>(base) + i) = q;
}
template <>
__device__ __forceinline__ void store_pairs4<float>(void* base, int64_t i, const float (&a)[4],
                                                    const float (&b)[4]) {
  f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(base) + 2 * i);
  o[0] = f32x4{a[0], b[0], a[1], b[1]};
  o[1] = f32x4{a[2], b[2], a[3], b[3]};
}
// The word holding one pair, for loads kept in registers before use.
template <typename T>
struct PairWord;
template <>
struct PairWord<bf16_t> {
  typedef uint32_t type;
  __device__ static __forceinline__ type zero() { return 0u; }
  __device__ static __forceinline__ void unpack(type v, float& a, float& b) {
    a = __uint_as_float(v << 16);
    b = __uint_as_float(v & 0xffff0000u);
  }
};
template <>
struct PairWord<float> {
  typedef float type __attribute__((ext_vector_type(2)));
  __device__ static __forceinline__ type zero() { return type{0.f, 0.f}; }
  __device__ static __forceinline__ void unpack(type v, float& a, float& b) {
    a = v.x;
    b = v.y;
  }
};

// SiLU(g) * u = g * u / (1 + e^-g) (SwiGLU, lesson 13, section 1.2), as
// g * u / (1 + 2^(-g log2 e)) with v_exp_f32 and v_rcp_f32 (about 1 ulp each).
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// Wavefront (64 lanes) reductions; the butterfly order is fixed, so results
// are identical run to run.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wavefront, with DPP lane
// moves (no LDS round trips): within each row of 16 lanes add the values
// shifted down by 1, 2, 4 and 8 lanes (lanes shifted in from outside the row
// add 0), then add the last lane of row 0 to row 1 and of row 2 to row 3
// (row_bcast:15), then lane 31 to rows 2 and 3 (row_bcast:31).  Integer
// sums, so the result does not depend on the order.
__device__ __forceinline__ int wave_inclusive_scan(int v, int /*lane*/) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
  return v;
}

}  // namespace topmoe
