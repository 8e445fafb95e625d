// Direct global -> LDS staging of 64-row 16-bit tiles (bf16 or fp16) for the
// gfx950 kernels.
//
// A tile holds 64 rows of D 16-bit values (row bytes RB = 2*D, no padding).  The 16-byte
// chunk c of row r is stored at chunk c ^ (r mod CH), CH = D/8 chunks per row:
// rows that an MFMA operand read touches at the same time land on different
// banks, for both the row-operand reads and the LDS transpose reads.
//
// Loads use buffer_load ... lds (lds_dma): lane l of a wave writes its 16 bytes
// to LDS base + 16*l, so one instruction fills 64/CH whole rows; the global chunk
// a lane fetches is chosen so that the row it fills ends up swizzled.  An
// out-of-range offset (padding row) writes zeros.  A wave stages its own 16
// rows of every tile; a ring of LDS stages lets the loads of several tiles be
// in flight (no registers hold them).
#pragma once

#include "st_device.hpp"

namespace st {

template <int D>
struct TileShape {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int RB = D * 2;                 // bytes per row
  static constexpr int BYTES = kBlock * RB;        // bytes per tile
  static constexpr int RPI = 64 / CH;              // rows filled by one wave instruction
  static constexpr int NI = 16 / RPI;              // instructions per wave per tile (16 rows)
  static_assert(NI >= 1 && 16 % RPI == 0, "tile shape");
  // byte offset of chunk c of row r inside a tile
  __device__ static __forceinline__ int phys(int r, int c) { return r * RB + ((c ^ (r & (CH - 1))) << 4); }
};

// LDS byte address of a __shared__ pointer, made wave-uniform.  A generic
// pointer into LDS holds the LDS offset in its low 32 bits (the high half is
// the shared aperture), so no address-space cast (and no null check) is needed.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)p);
}

// One buffer_load ... lds of BYTES (16 or 4) per lane: lane l's bytes land at
// LDS lds_base + BYTES*l.  Written as inline asm on purpose: the compiler's
// wait-count insertion cannot tell the ring stages apart and would make every
// LDS read wait for all DMA loads in flight, which serialises the ring; the
// kernels order these loads with their own s_waitcnt vmcnt + barrier instead.
// M0 carries the LDS base, and one wait state separates the M0 write from the
// load that reads it.  M0 is clobbered without being restored: nothing else in
// these kernels uses it (the compiler only would for LDS DMA builtins, GWS or
// message instructions, which they do not contain; a codegen test checks that
// M0 appears only inside these asm blocks).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int BYTES>
__device__ __forceinline__ void lds_dma(Rsrc r, uint32_t lds_base, uint32_t voff) {
  if constexpr (BYTES == 16) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(r)
                 : "memory", "m0");
  } else {
    static_assert(BYTES == 4, "16- or 4-byte DMA");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(r)
                 : "memory", "m0");
  }
}
#pragma clang diagnostic pop

// Stage N*RPI rows of one 64-row tile of a [T, D] 16-bit tensor (N = NI: the
// wave's 16 rows): `rows` is the wave-uniform LDS address of the first of them,
// tile row `row0`; pos[i] is the position for tile row row0 + i*RPI + lane/CH,
// or -1 for padding.  The chunk a lane fetches is the one that its LDS slot
// holds after the swizzle of its row (row mod CH).
template <int D, int N>
__device__ __forceinline__ void stage_rows(Rsrc src, uint32_t rows, int row0, int lane, const int (&pos)[N]) {
  using S = TileShape<D>;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int r = row0 + i * S::RPI + lane / S::CH;              // tile row this lane fills
    const int lc = (lane % S::CH) ^ (r & (S::CH - 1));           // logical chunk this lane fetches
    const uint32_t off = pos[i] >= 0 ? (uint32_t)(pos[i] * S::RB + lc * 16) : kOutOfRange;
    lds_dma<16>(src, rows + i * S::RPI * S::RB, off);
  }
}

// Wait until at most n vector-memory loads of this wave are outstanding
// (loads complete in issue order).  n is a compile-time constant.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] and [15:14]; expcnt[6:4] and lgkmcnt[11:8] left at their maximum
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Wait until this wave's LDS and scalar-memory operations have completed
// (lgkmcnt 0; vmcnt and expcnt left at their maximum).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// wait_vmcnt<per_tile * k> for a runtime k in [0, KMAX].
template <int PER_TILE, int KMAX>
__device__ __forceinline__ void wait_tiles_left(int k) {
  if constexpr (KMAX >= 3) {
    if (k >= 3) {
      wait_vmcnt<PER_TILE * 3>();
      return;
    }
  }
  if constexpr (KMAX >= 2) {
    if (k == 2) {
      wait_vmcnt<PER_TILE * 2>();
      return;
    }
  }
  if constexpr (KMAX >= 1) {
    if (k == 1) {
      wait_vmcnt<PER_TILE>();
      return;
    }
  }
  wait_vmcnt<0>();
}

}  // namespace st
