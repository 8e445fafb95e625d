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
//                 set of t is the class prefix [r*n_pad, R]
//   K_BLOCK       rows = keys = positions; [l*floor(t/l), t]
//   K_SUMMARY     compact summary keys b*c + o <-> b*l + (l-c) + o for blocks
//                 b < ceil(T/l) - 1; strictly earlier blocks: [0, c*floor(t/l) - 1]
//   K_SUMMARY_R1  compact summary keys of every block (positions >= T are
//                 padding); earlier blocks plus own-block summary keys <= t
//   K_CAUSAL      rows = keys = positions; [0, t]
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
};

constexpr int kBlock = 64;  // LUT block size, rows and keys

struct Geometry {
  int code;    // KindCode
  int T, l, c;
  int n_rows;  // kernel rows, padding included
  int n_keys;  // kernel keys, padding included
  int n_pad;   // K_STRIDE: class length rounded up to kBlock
  int n_cls;   // K_STRIDE: number of residue classes, min(l, T)
};

ST_HD int imin(int a, int b) { return a < b ? a : b; }
ST_HD int imax(int a, int b) { return a > b ? a : b; }

// Position held by kernel row R, or -1 for padding / out of range.
ST_HD int row_position(const Geometry& g, int R) {
  if (R < 0 || R >= g.n_rows) return -1;
  if (g.code == K_STRIDE) {
    const int r = R / g.n_pad;
    const int m = R - r * g.n_pad;
    const int64_t p = (int64_t)m * g.l + r;
    return p < g.T ? (int)p : -1;
  }
  return R;
}

// Position held by kernel key K, or -1 for padding / out of range.
ST_HD int key_position(const Geometry& g, int K) {
  if (K < 0 || K >= g.n_keys) return -1;
  if (g.code == K_STRIDE) {
    const int r = K / g.n_pad;
    const int m = K - r * g.n_pad;
    const int64_t p = (int64_t)m * g.l + r;
    return p < g.T ? (int)p : -1;
  }
  if (g.code == K_SUMMARY || g.code == K_SUMMARY_R1) {
    const int b = K / g.c;
    const int o = K - b * g.c;
    const int64_t p = (int64_t)b * g.l + (g.l - g.c) + o;
    return p < g.T ? (int)p : -1;
  }
  return K;
}

// True when position t of this kind is some kernel key (else nobody attends it).
ST_HD bool position_is_key(const Geometry& g, int t) {
  if (g.code == K_SUMMARY || g.code == K_SUMMARY_R1) {
    const int b = t / g.l;
    const int off = t - b * g.l;
    if (off < g.l - g.c) return false;
    return g.code == K_SUMMARY_R1 || (int64_t)(b + 1) * g.c <= g.n_keys;
  }
  return true;
}

// Run [lo, hi] of kernel keys attended by kernel row R holding position t >= 0.
// lo > hi means the row attends nothing.
ST_HD void row_interval(const Geometry& g, int R, int t, int& lo, int& hi) {
  switch (g.code) {
    case K_LOCAL:
      lo = imax(0, t - g.l + 1);
      hi = t;
      break;
    case K_STRIDE:
      lo = (R / g.n_pad) * g.n_pad;
      hi = R;
      break;
    case K_BLOCK:
      lo = (t / g.l) * g.l;
      hi = t;
      break;
    case K_SUMMARY:
      lo = 0;
      hi = g.c * (t / g.l) - 1;
      break;
    case K_SUMMARY_R1: {
      const int b = t / g.l;
      const int off = t - b * g.l;
      lo = 0;
      hi = g.c * b + imax(0, off - (g.l - g.c) + 1) - 1;
      break;
    }
    default:  // K_CAUSAL
      lo = 0;
      hi = t;
      break;
  }
}

}  // namespace st
