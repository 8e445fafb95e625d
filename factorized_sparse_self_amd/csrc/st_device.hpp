// Device helpers for the gfx950 (CDNA4) attention kernels: vector types,
// MFMA wrappers and the lane geometry every kernel shares.
//
// Wave layout.  A wave is 64 lanes; lane = 16*lg + li with li in [0,16) and
// lg in [0,4).  For the 16x16 MFMAs used here (v_mfma_f32_16x16x32_{bf16,f16} and
// v_mfma_f32_16x16x4_f32), with D[M][N] = sum_k A[M][k] B[k][N]:
//   A operand: lane holds A[M = li][k = kw*lg + (0..kw-1)]
//   B operand: lane holds B[k = kw*lg + (0..kw-1)][N = li]
//   C / D    : lane holds D[M = 4*lg + e][N = li], e = 0..3
// with kw = 8 (16-bit, K = 32) or kw = 1 (fp32, K = 4).  So a product whose N
// index is the lane's own query (or key) leaves that row's values in the
// lane, which keeps the softmax row reductions mostly inside a lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "st_geometry.hpp"

namespace st {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = 256;    // 4 waves per workgroup
constexpr int kDqThreads = 512;  // 16-bit dq: 8 waves, 16 rows each of a pair of row blocks

// 16-bit element types of the MFMA kernels (bf16, fp16) and their vectors.
template <typename E>
struct Vec;
template <>
struct Vec<bf16> {
  typedef bf16x8 x8;
  typedef bf16x4 x4;
  typedef bf16x2 x2;
};
template <>
struct Vec<f16> {
  typedef f16x8 x8;
  typedef f16x4 x4;
  typedef f16x2 x2;
};
template <typename TE>
struct Is16 {
  static constexpr bool value = std::is_same<TE, bf16>::value || std::is_same<TE, f16>::value;
};

// v_mfma_f32_16x16x32_{bf16,f16}: fp32 accumulation of 16-bit products.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Four fp32 values rounded to E (round-to-nearest-even), packed.
template <typename E>
__device__ __forceinline__ typename Vec<E>::x4 to_x4(const f32x4& x) {
  typedef typename Vec<E>::x2 V2;
  const V2 lo = __builtin_convertvector((f32x2){x[0], x[1]}, V2);
  const V2 hi = __builtin_convertvector((f32x2){x[2], x[3]}, V2);
  return (typename Vec<E>::x4){lo[0], lo[1], hi[0], hi[1]};
}

// Eight values for the B operand of a 32-key (or 32-query) MFMA step:
// slots 0..3 come from one 16-block's C fragment, slots 4..7 from the next.
template <typename E>
__device__ __forceinline__ typename Vec<E>::x8 pack_b_operand(const f32x4& a, const f32x4& b) {
  const typename Vec<E>::x4 x = to_x4<E>(a);
  const typename Vec<E>::x4 y = to_x4<E>(b);
  return (typename Vec<E>::x8){x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

template <typename V4>
__device__ __forceinline__ auto concat(const V4& a, const V4& b) {
  typedef decltype(a[0] + a[0]) El;
  typedef El V8 __attribute__((ext_vector_type(8)));
  return (V8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes that
// share lg, lane i receives element (i mod 4) of the 8-byte chunks addressed by
// lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.  If lane j addresses row
// r0 + j/4, columns c0 + 4*(j mod 4) of a row-major tile, lane i therefore gets
// column c0 + i of rows r0 .. r0 + 3: the transposed operand an MFMA needs,
// read from a tile stored untransposed.
template <typename E>
__device__ __forceinline__ typename Vec<E>::x4 lds_read_tr(const E* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_bit_cast(typename Vec<E>::x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

__device__ __forceinline__ bool wave_any(bool v) { return __ballot(v) != 0ull; }

// Output rows are written 16 bytes per lane, D/8 consecutive lanes per row,
// so that one instruction writes whole 128-byte lines (one row at D = 64, two
// adjacent rows at D = 32).  Rows written once and not read again in the step
// (dq, dk, dv, and the zero dk / dv rows of keys nobody attends) use
// non-temporal stores: streamed past the caches, they do not evict the lines
// of Q, K, V and dO still being read.  Non-temporal stores of 8-byte pieces of
// lines were slower than ordinary ones, so the pieces go through LDS first.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_zero16_nt(void* p) {
  __builtin_nontemporal_store((u32x4){0u, 0u, 0u, 0u}, (u32x4*)p);
}

// Whole-row output of a wave's rows through LDS.  An MFMA output tile leaves
// each row in four lanes, lane (li, lg) holding elements 16 d + 4 lg .. + 3 of
// row li, i.e. 8-byte pieces of a line.  RowStage puts a wave's NR rows (NR/16
// such tiles) into an LDS buffer of the wave at a padded stride, then reads
// them back as 16-byte chunks, D/8 consecutive lanes per row.
template <typename E, int D, int NR>
struct RowStage {
  static constexpr int RS = D + 8;             // row stride, elements (16 B of padding)
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int BYTES = NR * RS * (int)sizeof(E);
  static constexpr int ROUNDS = NR * CH / 64;  // chunks per lane
  static_assert(NR % 16 == 0 && (NR * CH) % 64 == 0, "whole chunks per lane");
  E* buf;
  __device__ __forceinline__ explicit RowStage(void* p) : buf((E*)p) {}
  // rows 16 g + li of the buffer from one tile's ND accumulators, times scale
  template <int ND>
  __device__ __forceinline__ void put(int g, int li, int lg, const f32x4* x, float scale) {
#pragma unroll
    for (int d = 0; d < ND; ++d)
      *(typename Vec<E>::x4*)(buf + (16 * g + li) * RS + 16 * d + 4 * lg) = to_x4<E>(x[d] * scale);
  }
  // chunk `round` of this lane: its row and the chunk's element offset
  __device__ __forceinline__ int row_of(int lane, int round) const { return (lane + 64 * round) / CH; }
  __device__ __forceinline__ int col_of(int lane, int round) const { return (lane + 64 * round) % CH * 8; }
  __device__ __forceinline__ u32x4 get(int lane, int round) const {
    return *(const u32x4*)(buf + row_of(lane, round) * RS + col_of(lane, round));
  }
};

// Read-only tables (LUTs, schedules) are read through the constant address
// space: a uniform load from it is a scalar load, so values such as a block
// index or its FULL flag stay in scalar registers and branches on them are
// scalar branches.
template <typename T>
using cptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ cptr<T> as_const(const T* p) {
  return (cptr<T>)p;
}

// The rows a thread stages from every 64-block: rows srow + i*RSTEP.  Their
// per-row address parts are computed once; per block only the uniform block
// part is added (or, for a summary map whose c does not divide the block,
// the position is computed directly).
template <int NLD, int RSTEP>
struct StageRows {
  int row[NLD], off[NLD];
  bool split;
  template <class G>
  __device__ __forceinline__ StageRows(const G& g, bool keys, int srow) {
    split = split_position_ok(g, keys);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      row[i] = srow + i * RSTEP;
      off[i] = split ? row_part(g, keys, row[i]).off : 0;
    }
  }
  template <class G>
  __device__ __forceinline__ void positions(const G& g, bool keys, int blk, int (&p)[NLD]) const {
    if (split) {
      const BlockPart bp = block_part(g, keys, blk);
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int q = (residue_major(g) && row[i] >= bp.split ? bp.base2 : bp.base) + off[i];
        p[i] = (row[i] < bp.limit && q < g.T) ? q : -1;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NLD; ++i) p[i] = block_position(g, keys, blk, row[i]);
    }
  }
};

// Load a (trivially copyable) struct from a read-only table with scalar loads.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "dword-sized struct");
  struct Words {
    uint32_t w[sizeof(T) / 4];
  } tmp;
  const cptr<uint32_t> q = (cptr<uint32_t>)p;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) tmp.w[i] = q[i];
  return __builtin_bit_cast(T, tmp);
}

// Make a wave-uniform value explicit (scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Buffer resource over `bytes` bytes from `base` (bytes < 2^31).  Loads whose
// offset lies outside the buffer return zeros, so padding rows need no branch.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(Rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
// The same, non-temporal (cache policy nt): for data read once and not again
// in the step, so that it does not displace lines that are.
__device__ __forceinline__ uint4 buf_load16_nt(Rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}
__device__ __forceinline__ float buf_load_f32(Rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// Value of lane (lane ^ m) of the wave (ds_bpermute; m < 64).
__device__ __forceinline__ int xor_shfl(int v, int m) {
  return __builtin_amdgcn_ds_bpermute((int)(((threadIdx.x & 63) ^ m) << 2), v);
}
__device__ __forceinline__ float xor_shfl(float v, int m) { return __int_as_float(xor_shfl(__float_as_int(v), m)); }

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

// One head kind on the device: geometry plus its LUT.  Besides the byte flags,
// each CSR / CSC entry is also packed as one dword, block index | FULL << 31,
// so that a kernel reads both with one scalar load (a byte read would come
// back in a vector register and make the FULL branch look divergent).
constexpr uint32_t kFullBit = 0x80000000u;
struct KindDev {
  Geometry geo;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const uint8_t* flags;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  const uint8_t* csc_flags;
  const uint32_t* csr_entry;  // col_idx | flags << 31
  const uint32_t* csc_entry;  // row_idx | csc_flags << 31
  // Row-block pairs (2p, 2p+1): the union of the two CSR rows, one dword per
  // key block: block | half-0 bits << 28 | half-1 bits << 30, where the two
  // bits of a half are kPairVisit (the row block visits the key block) and
  // kPairFull (it is FULL for that row block).
  const int32_t* pair_ptr;
  const uint32_t* pair_entry;
  const uint8_t* row_flags;  // [T] per position: RowFlag bits of the 16-bit dq
};
constexpr uint32_t kPairVisit = 1u, kPairFull = 2u, kPairBlockMask = 0x0fffffffu;

}  // namespace st
