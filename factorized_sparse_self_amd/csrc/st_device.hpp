// Device helpers for the gfx950 (CDNA4) attention kernels: vector types,
// MFMA wrappers and the lane geometry every kernel shares.
//
// Wave layout.  A wave is 64 lanes; lane = 16*lg + li with li in [0,16) and
// lg in [0,4).  For the 16x16 MFMAs used here (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32), with D[M][N] = sum_k A[M][k] B[k][N]:
//   A operand: lane holds A[M = li][k = kw*lg + (0..kw-1)]
//   B operand: lane holds B[k = kw*lg + (0..kw-1)][N = li]
//   C / D    : lane holds D[M = 4*lg + e][N = li], e = 0..3
// with kw = 8 (bf16, K = 32) or kw = 1 (fp32, K = 4).  So a product whose N
// index is the lane's own query (or key) leaves that row's values in the
// lane, which keeps the softmax row reductions mostly inside a lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "st_geometry.hpp"

namespace st {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = 256;  // 4 waves per workgroup

template <typename TE>
struct IsBf16 {
  static constexpr bool value = false;
};
template <>
struct IsBf16<bf16> {
  static constexpr bool value = true;
};

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Four fp32 values rounded to bf16 (round-to-nearest-even), packed.
__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& x) {
  const bf16x2 lo = __builtin_convertvector((f32x2){x[0], x[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){x[2], x[3]}, bf16x2);
  return (bf16x4){lo[0], lo[1], hi[0], hi[1]};
}

// Eight values for the B operand of a 32-key (or 32-query) MFMA step:
// slots 0..3 come from one 16-block's C fragment, slots 4..7 from the next.
__device__ __forceinline__ bf16x8 pack_b_operand(const f32x4& a, const f32x4& b) {
  const bf16x4 x = to_bf16x4(a);
  const bf16x4 y = to_bf16x4(b);
  return (bf16x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// The same eight values as a bf16 pair x = hi + lo: hi is x truncated to bf16
// and lo is the rounded remainder, so a product summed over both halves keeps
// about 16 significant bits of x instead of bf16's 8.
__device__ __forceinline__ void split_b_operand(const f32x4& a, const f32x4& b, bf16x8& hi,
                                                bf16x8& lo) {
  uint32_t hw[4];
  f32x4 ra, rb;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t a0 = __builtin_bit_cast(uint32_t, a[2 * i]);
    const uint32_t a1 = __builtin_bit_cast(uint32_t, a[2 * i + 1]);
    const uint32_t b0 = __builtin_bit_cast(uint32_t, b[2 * i]);
    const uint32_t b1 = __builtin_bit_cast(uint32_t, b[2 * i + 1]);
    hw[i] = (a0 >> 16) | (a1 & 0xffff0000u);
    hw[2 + i] = (b0 >> 16) | (b1 & 0xffff0000u);
    ra[2 * i] = a[2 * i] - __builtin_bit_cast(float, a0 & 0xffff0000u);
    ra[2 * i + 1] = a[2 * i + 1] - __builtin_bit_cast(float, a1 & 0xffff0000u);
    rb[2 * i] = b[2 * i] - __builtin_bit_cast(float, b0 & 0xffff0000u);
    rb[2 * i + 1] = b[2 * i + 1] - __builtin_bit_cast(float, b1 & 0xffff0000u);
  }
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  hi = __builtin_bit_cast(bf16x8, (u32x4){hw[0], hw[1], hw[2], hw[3]});
  lo = pack_b_operand(ra, rb);
}

__device__ __forceinline__ bf16x8 concat(const bf16x4& a, const bf16x4& b) {
  return (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ float xor_shfl(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int xor_shfl(int v, int m) { return __shfl_xor(v, m, 64); }

// Reduce over the four lanes that share li (lg = 0..3).
__device__ __forceinline__ float group4_max(float v) {
  v = fmaxf(v, xor_shfl(v, 16));
  return fmaxf(v, xor_shfl(v, 32));
}
__device__ __forceinline__ float group4_sum(float v) {
  v += xor_shfl(v, 16);
  return v + xor_shfl(v, 32);
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = imin(v, xor_shfl(v, m));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = imax(v, xor_shfl(v, m));
  return v;
}

// One head kind on the device: geometry plus its LUT.
struct KindDev {
  Geometry geo;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const uint8_t* flags;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  const uint8_t* csc_flags;
};

}  // namespace st
