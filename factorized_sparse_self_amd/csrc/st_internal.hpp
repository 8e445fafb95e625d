// Host-side internals shared by the layout builder and the C ABI.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "st_geometry.hpp"

namespace st {

struct KindLayout {
  Geometry geo;
  int n_qb = 0;
  int n_kb = 0;
  int64_t pairs = 0;  // attended (query, key) pairs of one head
  std::vector<int32_t> row_ptr, col_idx;
  std::vector<uint8_t> flags;
  std::vector<int32_t> col_ptr, row_idx;
  std::vector<uint8_t> csc_flags;
};

// True for the patterns with a summary kind (they take c and a summary set).
bool uses_summary(int pattern);

// Fill the geometry of (pattern, kind); returns false on an unknown pattern.
// sigma: the summary offsets (null for the last c); the geometry keeps the
// pointer, which must outlive it.
bool make_geometry(int pattern, int kind, int T, int l, int c, const int32_t* sigma, Geometry* g);

// Argument check shared by st_layout_build and the attention calls (summary:
// null, or c strictly ascending offsets in [0, l) for a summary pattern).
// Returns an empty string when valid, else the reason.
std::string check_pattern_args(int pattern, int T, int l, int c, const int32_t* summary);

// The summary set as stored: empty for the default set (the last c offsets,
// whether given or not), else the c offsets.
std::vector<int32_t> canonical_summary(int pattern, int l, int c, const int32_t* summary);

// Build the CSR / CSC of one kind (the geometry must already be set).
void build_kind(KindLayout& L);

// Thread-local last-error message.
void set_error(const std::string& msg);

}  // namespace st

struct st_layout {
  int pattern, T, l, c;
  std::vector<int32_t> summary;  // non-default summary offsets (the geometries point here)
  st::KindLayout kind[2];
};
