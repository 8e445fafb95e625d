// Host check of the layout builder's memory safety (built with AddressSanitizer
// and UndefinedBehaviorSanitizer by the test that runs it; CPU only).
//
// Builds the layouts of every pattern over a grid of (T, l, c) and summary
// sets, ragged and degenerate ones included, copies every table out into
// buffers of exactly the advertised sizes, and checks the tables' structure:
// monotone pointers, indices in range, CSR and CSC listing the same pairs with
// the same flags, and every listed block pair inside the maps.  Invalid
// arguments must be refused without touching memory.  Prints "ok <count>".
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <tuple>
#include <vector>

#include "st.h"

namespace {

int g_fail = 0;
long g_checked = 0;

void fail(const char* what, int pattern, int T, int l, int c, int kind) {
  if (g_fail < 20) printf("FAIL %s: pattern %d T %d l %d c %d kind %d\n", what, pattern, T, l, c, kind);
  ++g_fail;
}

void check_kind(const st_layout* lay, int kind, int pattern, int T, int l, int c) {
  int32_t dims[ST_DIM_COUNT];
  if (st_layout_dims(lay, kind, dims) != ST_OK) return fail("dims", pattern, T, l, c, kind);
  const int B = dims[ST_DIM_BLOCK], rows = dims[ST_DIM_ROWS], keys = dims[ST_DIM_KEYS];
  const int nq = dims[ST_DIM_QBLOCKS], nk = dims[ST_DIM_KBLOCKS], nnz = dims[ST_DIM_NNZ];
  if (B <= 0 || rows < 0 || keys < 0 || nq != (rows + B - 1) / B || nk != (keys + B - 1) / B || nnz < 0 ||
      (int64_t)nnz > (int64_t)nq * nk)
    return fail("dims values", pattern, T, l, c, kind);
  int64_t pairs = -1;
  if (st_layout_pairs(lay, kind, &pairs) != ST_OK || pairs < 0) return fail("pairs", pattern, T, l, c, kind);
  // exact-size heap buffers: a write past any of them is reported
  std::vector<int32_t> row_pos(rows), key_pos(keys);
  if (st_layout_maps(lay, kind, row_pos.data(), row_pos.size(), key_pos.data(), key_pos.size()) != ST_OK)
    return fail("maps", pattern, T, l, c, kind);
  for (int32_t p : row_pos)
    if (p < -1 || p >= T) return fail("row map range", pattern, T, l, c, kind);
  for (int32_t p : key_pos)
    if (p < -1 || p >= T) return fail("key map range", pattern, T, l, c, kind);
  std::vector<int32_t> row_ptr(nq + 1), col_idx(nnz), col_ptr(nk + 1), row_idx(nnz);
  std::vector<uint8_t> cflags(nnz), kflags(nnz);
  if (st_layout_csr(lay, kind, row_ptr.data(), row_ptr.size(), col_idx.data(), col_idx.size(), cflags.data(),
                    cflags.size()) != ST_OK)
    return fail("csr", pattern, T, l, c, kind);
  if (st_layout_csc(lay, kind, col_ptr.data(), col_ptr.size(), row_idx.data(), row_idx.size(), kflags.data(),
                    kflags.size()) != ST_OK)
    return fail("csc", pattern, T, l, c, kind);
  // one element short in any buffer: refused, nothing written
  {
    if (st_layout_csr(lay, kind, row_ptr.data(), row_ptr.size() - 1, col_idx.data(), col_idx.size(), cflags.data(),
                      cflags.size()) != ST_ERR_BUFFER_TOO_SMALL)
      return fail("csr short row_ptr", pattern, T, l, c, kind);
  }
  if (nnz > 0) {
    if (st_layout_csc(lay, kind, col_ptr.data(), col_ptr.size(), row_idx.data(), row_idx.size() - 1, kflags.data(),
                      kflags.size()) != ST_ERR_BUFFER_TOO_SMALL)
      return fail("csc short row_idx", pattern, T, l, c, kind);
  }
  if (rows > 0) {
    if (st_layout_maps(lay, kind, row_pos.data(), row_pos.size() - 1, key_pos.data(), key_pos.size()) !=
        ST_ERR_BUFFER_TOO_SMALL)
      return fail("maps short row_pos", pattern, T, l, c, kind);
  }
  if (row_ptr[0] != 0 || row_ptr[nq] != nnz || col_ptr[0] != 0 || col_ptr[nk] != nnz)
    return fail("pointer ends", pattern, T, l, c, kind);
  std::vector<std::tuple<int, int, int>> a, b;  // (row block, key block, flag)
  for (int qb = 0; qb < nq; ++qb) {
    if (row_ptr[qb] > row_ptr[qb + 1]) return fail("csr monotone", pattern, T, l, c, kind);
    for (int e = row_ptr[qb]; e < row_ptr[qb + 1]; ++e) {
      if (col_idx[e] < 0 || col_idx[e] >= nk || (e > row_ptr[qb] && col_idx[e] <= col_idx[e - 1]))
        return fail("csr index", pattern, T, l, c, kind);
      a.emplace_back(qb, col_idx[e], cflags[e]);
    }
  }
  for (int kb = 0; kb < nk; ++kb) {
    if (col_ptr[kb] > col_ptr[kb + 1]) return fail("csc monotone", pattern, T, l, c, kind);
    for (int e = col_ptr[kb]; e < col_ptr[kb + 1]; ++e) {
      if (row_idx[e] < 0 || row_idx[e] >= nq || (e > col_ptr[kb] && row_idx[e] <= row_idx[e - 1]))
        return fail("csc index", pattern, T, l, c, kind);
      b.emplace_back(row_idx[e], kb, kflags[e]);
    }
  }
  std::sort(b.begin(), b.end());
  if (a != b) return fail("csr and csc differ", pattern, T, l, c, kind);
  ++g_checked;
}

void check(int pattern, int T, int l, int c, const int32_t* summary) {
  st_layout* lay = nullptr;
  const int rc = summary ? st_layout_build_ex(pattern, T, l, c, summary, &lay) : st_layout_build(pattern, T, l, c, &lay);
  if (rc != ST_OK || !lay) return fail("build", pattern, T, l, c, -1);
  check_kind(lay, 0, pattern, T, l, c);
  check_kind(lay, 1, pattern, T, l, c);
  // out-of-range kinds are refused
  int32_t dims[ST_DIM_COUNT];
  if (st_layout_dims(lay, 2, dims) == ST_OK || st_layout_dims(lay, -1, dims) == ST_OK)
    fail("kind range", pattern, T, l, c, 2);
  st_layout_free(lay);
}

}  // namespace

int main() {
  const int patterns[] = {ST_STRIDED, ST_FIXED, ST_FIXED_R1, ST_DENSE, ST_STRIDED_UNION, ST_FIXED_UNION};
  const int Ts[] = {1, 2, 7, 63, 64, 65, 127, 128, 129, 250, 333, 1000, 4096};
  const int ls[] = {1, 2, 3, 5, 16, 20, 63, 64, 65, 128, 500, 5000};
  for (int pattern : patterns)
    for (int T : Ts)
      for (int l : ls) {
        const bool summary = pattern == ST_FIXED || pattern == ST_FIXED_R1 || pattern == ST_FIXED_UNION;
        if (!summary) {
          check(pattern, T, l, 0, nullptr);
          continue;
        }
        for (int c : {1, 2, l / 2, l - 1, l})
          if (c >= 1 && c <= l) check(pattern, T, l, c, nullptr);
        // explicit summary sets: first offset, spread offsets, every offset
        std::vector<int32_t> s1 = {0}, s2, s3;
        for (int o = 0; o < l; o += 3) s2.push_back(o);
        for (int o = 0; o < l; ++o) s3.push_back(o);
        check(pattern, T, l, (int)s1.size(), s1.data());
        check(pattern, T, l, (int)s2.size(), s2.data());
        if (l <= 500) check(pattern, T, l, (int)s3.size(), s3.data());
      }
  // invalid arguments are refused and leave *out untouched
  st_layout* lay = nullptr;
  const int32_t bad_set[] = {3, 1};
  const int32_t out_of_block[] = {0, 16};
  struct Bad {
    int pattern, T, l, c;
    const int32_t* summary;
  } bad[] = {{ST_STRIDED, 0, 16, 0, nullptr},   {ST_STRIDED, -5, 16, 0, nullptr},
             {ST_STRIDED, 100, 0, 0, nullptr},  {ST_FIXED, 100, 16, 0, nullptr},
             {ST_FIXED, 100, 16, 17, nullptr},  {ST_FIXED, (1 << 24) + 1, 16, 4, nullptr},
             {ST_FIXED, 100, 16, 2, bad_set},   {ST_FIXED, 100, 16, 2, out_of_block},
             {ST_STRIDED, 100, 16, 1, bad_set}, {99, 100, 16, 4, nullptr},
             {-1, 100, 16, 4, nullptr}};
  for (const Bad& x : bad) {
    const int rc = x.summary ? st_layout_build_ex(x.pattern, x.T, x.l, x.c, x.summary, &lay)
                             : st_layout_build(x.pattern, x.T, x.l, x.c, &lay);
    if (rc == ST_OK || lay != nullptr) fail("invalid arguments accepted", x.pattern, x.T, x.l, x.c, -1);
  }
  if (g_fail) {
    printf("%d failures\n", g_fail);
    return 1;
  }
  printf("ok %ld\n", g_checked);
  return 0;
}
