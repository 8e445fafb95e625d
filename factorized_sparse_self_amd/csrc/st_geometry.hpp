// Kernel coordinates of one head kind: the row / key maps and the run of
// kernel keys each kernel row attends.  Shared by the host LUT builder and
// the device kernels, so that the LUT and the in-tile masks agree exactly.
//
// The key sets follow llm-arch-kb "Sparse Transformer", §2 Derivation
// (Pattern A -- strided, Pattern B -- fixed) and nlp-lineage, "The idea"
// (one sub-pattern per head).  The maps are chosen so that every kernel row
// attends a single contiguous run [lo, hi] of kernel keys:
//   K_LOCAL       rows = keys = positions; [max(0, t-l+1), t]
//   K_STRIDE      residue-major: position m*l + r <-> r*n_pad + m; the strided
//                 set of t is the class prefix [r*n_pad, R].  n_pad is the
//                 class length rounded up to kClassGran = kBlock / 2, so a
//                 64-block holds one class, or the tail of one and the head
//                 of the next (96-long classes fill 64-blocks three to two)
//   K_BLOCK       rows = keys = positions; [l*floor(t/l), t]
//   K_SUMMARY     compact summary keys b*c + o <-> b*l + S[o] for blocks
//                 b < ceil(T/l) - 1, S the summary offsets (by default the last
//                 c: S[o] = l - c + o); strictly earlier blocks: [0, c*floor(t/l) - 1]
//   K_SUMMARY_R1  compact summary keys of every block (positions >= T are
//                 padding); earlier blocks plus own-block summary keys <= t
//   K_CAUSAL      rows = keys = positions; [0, t]
//   K_STRIDE_X    K_STRIDE without the row's own key: [r*n_pad, R-1] (the
//                 strided pass of a merged head, whose window holds t)
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define ST_HD __host__ __device__ __forceinline__
#else
#define ST_HD inline
#endif

namespace st {

enum KindCode : int {
  K_LOCAL = 0,
  K_STRIDE = 1,
  K_BLOCK = 2,
  K_SUMMARY = 3,
  K_SUMMARY_R1 = 4,
  K_CAUSAL = 5,
  K_STRIDE_X = 6,
};

constexpr int kBlock = 64;  // LUT block size, rows and keys
constexpr int kClassGran = kBlock / 2;  // residue-major class padding granule

// Division of a non-negative int by a fixed divisor as multiply-shift
// (Granlund and Montgomery, 1994): with s = 31 + ceil(log2 d) and
// m = ceil(2^s / d) (< 2^32), m*d - 2^s < d <= 2^(s-31), so
// floor(n*m / 2^s) == floor(n / d) for every 0 <= n < 2^31.
struct FastDiv {
  uint32_t mul, shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t lg = 0;
  while ((1ull << lg) < d) ++lg;
  const uint32_t s = 31 + lg;
  return {(uint32_t)(((1ull << s) + d - 1) / d), s};
}
ST_HD int fdiv(int n, FastDiv f) { return (int)(((uint64_t)(uint32_t)n * f.mul) >> f.shift); }

struct Geometry {
  int code;    // KindCode
  int T, l, c;
  int n_rows;  // kernel rows, padding included
  int n_keys;  // kernel keys, padding included
  int n_pad;   // K_STRIDE: class length rounded up to kClassGran
  int n_cls;   // K_STRIDE: number of residue classes, min(l, T)
  FastDiv div_l, div_c, div_pad;  // division by l, c (>= 1) and n_pad (>= 1)
  int blk_c;   // kBlock / c when c divides kBlock (summary blocks per LUT block), else 0
  const int32_t* sigma;  // summary kinds: the c offsets of S, ascending (host or device
                         // memory, as the geometry's user); null: the last c offsets
};

// A Geometry whose kind code is a compile-time constant.  The functions below
// are templates over the geometry type: called with a GeoC, every branch on the
// code folds away (the device kernels are instantiated per kind code); called
// with a plain Geometry, the code is read at run time (host LUT builder).
template <int KC>
struct GeoC : Geometry {
  static constexpr int code = KC;
};

ST_HD int imin(int a, int b) { return a < b ? a : b; }
ST_HD int imax(int a, int b) { return a > b ? a : b; }

// Residue-major maps (K_STRIDE and K_STRIDE_X share them).
template <class G>
ST_HD bool residue_major(const G& g) {
  return g.code == K_STRIDE || g.code == K_STRIDE_X;
}

// Summary set S of a summary kind: offset of its o-th element, the number of
// elements <= off, and membership (off in [0, l)).
template <class G>
ST_HD int summary_offset(const G& g, int o) {
  return g.sigma ? g.sigma[o] : g.l - g.c + o;
}
template <class G>
ST_HD int summary_count(const G& g, int off) {
  if (!g.sigma) return imax(0, off - (g.l - g.c) + 1);
  int lo = 0, hi = g.c;  // first element > off
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (g.sigma[mid] <= off)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}
template <class G>
ST_HD bool summary_member(const G& g, int off) {
  if (!g.sigma) return off >= g.l - g.c;
  const int n = summary_count(g, off);
  return n > 0 && g.sigma[n - 1] == off;
}

// Position held by kernel row R, or -1 for padding / out of range.
template <class G>
ST_HD int row_position(const G& g, int R) {
  if (R < 0 || R >= g.n_rows) return -1;
  if (residue_major(g)) {
    const int r = fdiv(R, g.div_pad);
    const int m = R - r * g.n_pad;
    const int64_t p = (int64_t)m * g.l + r;
    return p < g.T ? (int)p : -1;
  }
  return R;
}

// Position held by kernel key K, or -1 for padding / out of range.
template <class G>
ST_HD int key_position(const G& g, int K) {
  if (K < 0 || K >= g.n_keys) return -1;
  if (residue_major(g)) {
    const int r = fdiv(K, g.div_pad);
    const int m = K - r * g.n_pad;
    const int64_t p = (int64_t)m * g.l + r;
    return p < g.T ? (int)p : -1;
  }
  if (g.code == K_SUMMARY || g.code == K_SUMMARY_R1) {
    const int b = fdiv(K, g.div_c);
    const int o = K - b * g.c;
    const int64_t p = (int64_t)b * g.l + summary_offset(g, o);
    return p < g.T ? (int)p : -1;
  }
  return K;
}

// Position held by row i (0 <= i < kBlock) of 64-block `blk` of the kernel rows
// (keys == false) or kernel keys (keys == true); -1 for padding.  The branch on
// the kind is uniform; only the compact summary map divides, by multiply-shift.
template <class G>
ST_HD int block_position(const G& g, bool keys, int blk, int i) {
  const int R = blk * kBlock + i;
  if (residue_major(g)) {
    const int cls = fdiv(R, g.div_pad);
    const int p = (R - cls * g.n_pad) * g.l + cls;
    return (cls < g.n_cls && p < g.T) ? p : -1;
  }
  if (keys && (g.code == K_SUMMARY || g.code == K_SUMMARY_R1)) {
    if (R >= g.n_keys) return -1;
    const int q = fdiv(R, g.div_c);
    const int p = q * g.l + summary_offset(g, R - q * g.c);
    return p < g.T ? p : -1;
  }
  return R < g.T ? R : -1;
}

// block_position() split into a part that depends only on the block (uniform)
// and a part that depends only on the row offset i (per thread, fixed for a
// kernel's staging rows): position = (i < split ? base : base2) + off, valid
// iff i < limit and position < T.  Only a residue-major block has split <
// kBlock: its rows from `split` on belong to the next class.  Available when
// the map allows it: always for the identity and residue-major maps, and for
// the compact summary map when c divides kBlock.
struct RowPart {
  int off;
};
struct BlockPart {
  int base, limit, split, base2;
};
template <class G>
ST_HD bool split_position_ok(const G& g, bool keys) {
  return !(keys && (g.code == K_SUMMARY || g.code == K_SUMMARY_R1)) || (kBlock % g.c) == 0;
}
template <class G>
ST_HD RowPart row_part(const G& g, bool keys, int i) {
  if (residue_major(g)) return {i * g.l};
  if (keys && (g.code == K_SUMMARY || g.code == K_SUMMARY_R1)) {
    const int q = fdiv(i, g.div_c);
    return {q * g.l + summary_offset(g, i - q * g.c)};
  }
  return {i};
}
template <class G>
ST_HD BlockPart block_part(const G& g, bool keys, int blk) {
  if (residue_major(g)) {
    // rows [0, split) hold class cls from index m0 on; n_pad and m0 are
    // multiples of kClassGran, so split >= kClassGran and the remaining
    // kBlock - split <= n_pad rows hold class cls + 1 from index 0:
    // position (i - split) * l + cls + 1 = i * l + base2
    const int cls = fdiv(blk * kBlock, g.div_pad);
    const int m0 = blk * kBlock - cls * g.n_pad;
    const int split = imin(kBlock, g.n_pad - m0);
    const int limit = cls >= g.n_cls ? 0 : (cls + 1 >= g.n_cls ? split : kBlock);
    return {m0 * g.l + cls, limit, split, cls + 1 - split * g.l};
  }
  if (keys && (g.code == K_SUMMARY || g.code == K_SUMMARY_R1))
    return {blk * g.blk_c * g.l, g.n_keys - blk * kBlock, kBlock, 0};
  return {blk * kBlock, kBlock, kBlock, 0};
}

// True when position t of this kind is some kernel key (else nobody attends it).
template <class G>
ST_HD bool position_is_key(const G& g, int t) {
  if (g.code == K_SUMMARY || g.code == K_SUMMARY_R1) {
    const int b = fdiv(t, g.div_l);
    const int off = t - b * g.l;
    if (!summary_member(g, off)) return false;
    return g.code == K_SUMMARY_R1 || (int64_t)(b + 1) * g.c <= g.n_keys;
  }
  return true;
}

// Run [lo, hi] of kernel keys attended by kernel row R holding position t >= 0.
// lo > hi means the row attends nothing.
template <class G>
ST_HD void row_interval(const G& g, int R, int t, int& lo, int& hi) {
  switch (g.code) {
    case K_LOCAL:
      lo = imax(0, t - g.l + 1);
      hi = t;
      break;
    case K_STRIDE:
      lo = fdiv(R, g.div_pad) * g.n_pad;
      hi = R;
      break;
    case K_STRIDE_X:
      lo = fdiv(R, g.div_pad) * g.n_pad;
      hi = R - 1;
      break;
    case K_BLOCK:
      lo = fdiv(t, g.div_l) * g.l;
      hi = t;
      break;
    case K_SUMMARY:
      lo = 0;
      hi = g.c * fdiv(t, g.div_l) - 1;
      break;
    case K_SUMMARY_R1: {
      const int b = fdiv(t, g.div_l);
      const int off = t - b * g.l;
      lo = 0;
      hi = g.c * b + summary_count(g, off) - 1;
      break;
    }
    default:  // K_CAUSAL
      lo = 0;
      hi = t;
      break;
  }
}

}  // namespace st
