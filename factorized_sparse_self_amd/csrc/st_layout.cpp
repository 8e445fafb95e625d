// Block LUT builder (host only, no GPU calls).
//
// The pages precompute each query's key indices and compute only the
// non-empty blocks of the attention matrix (llm-arch-kb "Sparse Transformer",
// §2 "Per-layer cost" and §3 Reference implementation).  Here every kernel row
// of a kind attends one contiguous run of kernel keys (st_geometry.hpp), so a
// row block's candidate key blocks are the span of its rows' runs and the
// pair count of each (row block, key block) is a sum of run/block overlaps:
// no per-pair enumeration is needed.
#include <algorithm>
#include <climits>
#include <cstring>
#include <new>
#include <string>

#include "../../include/st.h"
#include "st_internal.hpp"

namespace st {

namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string& msg) { g_last_error = msg; }

static const char* last_error_cstr() { return g_last_error.c_str(); }

bool uses_summary(int pattern) {
  return pattern == ST_FIXED || pattern == ST_FIXED_R1 || pattern == ST_FIXED_UNION;
}

bool make_geometry(int pattern, int kind, int T, int l, int c, const int32_t* sigma, Geometry* g) {
  g->sigma = sigma;
  g->T = T;
  g->l = l;
  g->c = c;
  g->n_pad = 0;
  g->n_cls = 0;
  switch (pattern) {
    case ST_STRIDED: g->code = kind ? K_STRIDE : K_LOCAL; break;
    case ST_FIXED: g->code = kind ? K_SUMMARY : K_BLOCK; break;
    case ST_FIXED_R1: g->code = kind ? K_SUMMARY_R1 : K_BLOCK; break;
    case ST_DENSE: g->code = K_CAUSAL; break;
    case ST_STRIDED_UNION: g->code = kind ? K_STRIDE_X : K_LOCAL; break;
    case ST_FIXED_UNION: g->code = kind ? K_SUMMARY : K_BLOCK; break;
    default: return false;
  }
  g->n_rows = T;
  g->n_keys = T;
  const int nb = (T + l - 1) / l;  // l-blocks, last one possibly short
  if (g->code == K_STRIDE || g->code == K_STRIDE_X) {
    g->n_pad = (nb + kClassGran - 1) / kClassGran * kClassGran;
    g->n_cls = l < T ? l : T;
    g->n_rows = g->n_cls * g->n_pad;
    g->n_keys = g->n_rows;
  } else if (g->code == K_SUMMARY) {
    g->n_keys = (nb - 1) * c;
  } else if (g->code == K_SUMMARY_R1) {
    g->n_keys = nb * c;
  }
  g->div_l = make_fastdiv((uint32_t)l);
  g->div_c = make_fastdiv(c > 0 ? (uint32_t)c : 1u);
  g->div_pad = make_fastdiv(g->n_pad > 0 ? (uint32_t)g->n_pad : 1u);
  g->blk_c = (c > 0 && kBlock % c == 0) ? kBlock / c : 0;
  return true;
}

std::string check_pattern_args(int pattern, int T, int l, int c, const int32_t* summary) {
  if (pattern < ST_STRIDED || pattern > ST_FIXED_UNION) return "unknown pattern " + std::to_string(pattern);
  if (T < 1 || T > (1 << 24)) return "T must be in [1, 2^24], got " + std::to_string(T);
  if (l < 1 || l > (1 << 24)) return "l must be in [1, 2^24], got " + std::to_string(l);
  if (uses_summary(pattern) && (c < 1 || c > l))
    return "c must be in [1, l] for the fixed patterns, got c=" + std::to_string(c) +
           " l=" + std::to_string(l);
  if (summary) {
    if (!uses_summary(pattern)) return "a summary set is only taken by the fixed patterns";
    for (int o = 0; o < c; ++o) {
      if (summary[o] < 0 || summary[o] >= l)
        return "summary offset " + std::to_string(summary[o]) + " is not in [0, l)";
      if (o > 0 && summary[o] <= summary[o - 1]) return "summary offsets must be strictly ascending";
    }
  }
  return std::string();
}

std::vector<int32_t> canonical_summary(int pattern, int l, int c, const int32_t* summary) {
  if (!summary || !uses_summary(pattern)) return {};
  bool tail = true;
  for (int o = 0; o < c; ++o) tail = tail && summary[o] == l - c + o;
  if (tail) return {};
  return std::vector<int32_t>(summary, summary + c);
}

void build_kind(KindLayout& L) {
  const Geometry& g = L.geo;
  const int bs = kBlock;
  L.n_qb = (g.n_rows + bs - 1) / bs;
  L.n_kb = (g.n_keys + bs - 1) / bs;
  L.pairs = 0;
  L.row_ptr.assign(L.n_qb + 1, 0);
  L.col_idx.clear();
  L.flags.clear();
  int lo[kBlock], hi[kBlock];
  for (int qb = 0; qb < L.n_qb; ++qb) {
    int kmin = INT_MAX, kmax = -1;
    for (int i = 0; i < bs; ++i) {
      const int R = qb * bs + i;
      const int t = row_position(g, R);
      lo[i] = 1;
      hi[i] = 0;
      if (t < 0) continue;
      row_interval(g, R, t, lo[i], hi[i]);
      if (lo[i] > hi[i]) continue;
      L.pairs += hi[i] - lo[i] + 1;
      kmin = std::min(kmin, lo[i]);
      kmax = std::max(kmax, hi[i]);
    }
    if (kmax >= 0) {
      for (int kb = kmin / bs; kb <= kmax / bs; ++kb) {
        const int k0 = kb * bs, k1 = k0 + bs - 1;
        int count = 0;
        for (int i = 0; i < bs; ++i) {
          const int a = std::max(lo[i], k0), b = std::min(hi[i], k1);
          if (a <= b) count += b - a + 1;
        }
        if (count > 0) {
          L.col_idx.push_back(kb);
          L.flags.push_back(count == bs * bs ? 1 : 0);
        }
      }
    }
    L.row_ptr[qb + 1] = (int32_t)L.col_idx.size();
  }
  // CSC by a counting sort over key blocks; row blocks stay ascending.
  const size_t nnz = L.col_idx.size();
  L.col_ptr.assign(L.n_kb + 1, 0);
  for (size_t e = 0; e < nnz; ++e) L.col_ptr[L.col_idx[e] + 1]++;
  for (int kb = 0; kb < L.n_kb; ++kb) L.col_ptr[kb + 1] += L.col_ptr[kb];
  L.row_idx.assign(nnz, 0);
  L.csc_flags.assign(nnz, 0);
  std::vector<int32_t> fill(L.col_ptr.begin(), L.col_ptr.end() - 1);
  for (int qb = 0; qb < L.n_qb; ++qb) {
    for (int e = L.row_ptr[qb]; e < L.row_ptr[qb + 1]; ++e) {
      const int dst = fill[L.col_idx[e]]++;
      L.row_idx[dst] = qb;
      L.csc_flags[dst] = L.flags[e];
    }
  }
}

}  // namespace st

using namespace st;

extern "C" {

static int layout_build(const char* fn, int pattern, int T, int l, int c, const int32_t* summary,
                        st_layout** out) {
  if (!out) {
    set_error(std::string(fn) + ": out is null");
    return ST_ERR_INVALID;
  }
  *out = nullptr;
  const std::string why = check_pattern_args(pattern, T, l, c, summary);
  if (!why.empty()) {
    set_error(std::string(fn) + ": " + why);
    return ST_ERR_INVALID;
  }
  st_layout* lay = new (std::nothrow) st_layout;
  if (!lay) {
    set_error("st_layout_build: out of host memory");
    return ST_ERR_NOMEM;
  }
  lay->pattern = pattern;
  lay->T = T;
  lay->l = l;
  lay->c = uses_summary(pattern) ? c : 0;
  try {
    lay->summary = canonical_summary(pattern, l, c, summary);
    const int32_t* sigma = lay->summary.empty() ? nullptr : lay->summary.data();
    for (int kind = 0; kind < 2; ++kind) {
      make_geometry(pattern, kind, T, l, lay->c, sigma, &lay->kind[kind].geo);
      build_kind(lay->kind[kind]);
    }
  } catch (const std::bad_alloc&) {
    delete lay;
    set_error(std::string(fn) + ": out of host memory");
    return ST_ERR_NOMEM;
  }
  *out = lay;
  return ST_OK;
}

int st_layout_build(int pattern, int T, int l, int c, st_layout** out) {
  return layout_build("st_layout_build", pattern, T, l, c, nullptr, out);
}

int st_layout_build_ex(int pattern, int T, int l, int c, const int32_t* summary, st_layout** out) {
  return layout_build("st_layout_build_ex", pattern, T, l, c, summary, out);
}

static const KindLayout* kind_of(const st_layout* lay, int kind, const char* fn) {
  if (!lay || (kind != 0 && kind != 1)) {
    set_error(std::string(fn) + ": null layout or kind not 0/1");
    return nullptr;
  }
  return &lay->kind[kind];
}

int st_layout_dims(const st_layout* lay, int kind, int32_t* dims) {
  const KindLayout* L = kind_of(lay, kind, "st_layout_dims");
  if (!L || !dims) {
    if (L) set_error("st_layout_dims: dims is null");
    return ST_ERR_INVALID;
  }
  dims[ST_DIM_BLOCK] = kBlock;
  dims[ST_DIM_ROWS] = L->geo.n_rows;
  dims[ST_DIM_KEYS] = L->geo.n_keys;
  dims[ST_DIM_QBLOCKS] = L->n_qb;
  dims[ST_DIM_KBLOCKS] = L->n_kb;
  dims[ST_DIM_NNZ] = (int32_t)L->col_idx.size();
  return ST_OK;
}

int st_layout_pairs(const st_layout* lay, int kind, int64_t* pairs) {
  const KindLayout* L = kind_of(lay, kind, "st_layout_pairs");
  if (!L || !pairs) {
    if (L) set_error("st_layout_pairs: pairs is null");
    return ST_ERR_INVALID;
  }
  *pairs = L->pairs;
  return ST_OK;
}

// A caller buffer for n elements: `cap` (in elements) must hold them, and the
// pointer may be null only when n is 0.  Nothing is written on failure.
static int check_out(const char* fn, const char* what, const void* p, size_t cap, size_t n) {
  if (n > 0 && !p) {
    set_error(std::string(fn) + ": " + what + " is null");
    return ST_ERR_INVALID;
  }
  if (cap < n) {
    set_error(std::string(fn) + ": " + what + " holds " + std::to_string(cap) + " elements, needs " +
              std::to_string(n));
    return ST_ERR_BUFFER_TOO_SMALL;
  }
  return ST_OK;
}

int st_layout_maps(const st_layout* lay, int kind, int32_t* row_pos, size_t row_pos_cap, int32_t* key_pos,
                   size_t key_pos_cap) {
  const char* fn = "st_layout_maps";
  const KindLayout* L = kind_of(lay, kind, fn);
  if (!L) return ST_ERR_INVALID;
  int rc = check_out(fn, "row_pos", row_pos, row_pos_cap, (size_t)L->geo.n_rows);
  if (rc == ST_OK) rc = check_out(fn, "key_pos", key_pos, key_pos_cap, (size_t)L->geo.n_keys);
  if (rc != ST_OK) return rc;
  for (int R = 0; R < L->geo.n_rows; ++R) row_pos[R] = row_position(L->geo, R);
  for (int K = 0; K < L->geo.n_keys; ++K) key_pos[K] = key_position(L->geo, K);
  return ST_OK;
}

// CSR or CSC copy-out: ptr[n_blocks + 1], idx[nnz], flags[nnz].
static int copy_sparse(const char* fn, const std::vector<int32_t>& ptr_src, const std::vector<int32_t>& idx_src,
                       const std::vector<uint8_t>& flag_src, int32_t* ptr, size_t ptr_cap, int32_t* idx,
                       size_t idx_cap, uint8_t* flags, size_t flags_cap) {
  int rc = check_out(fn, "pointer array", ptr, ptr_cap, ptr_src.size());
  if (rc == ST_OK) rc = check_out(fn, "index array", idx, idx_cap, idx_src.size());
  if (rc == ST_OK) rc = check_out(fn, "flags", flags, flags_cap, flag_src.size());
  if (rc != ST_OK) return rc;
  std::memcpy(ptr, ptr_src.data(), ptr_src.size() * sizeof(int32_t));
  if (!idx_src.empty()) {
    std::memcpy(idx, idx_src.data(), idx_src.size() * sizeof(int32_t));
    std::memcpy(flags, flag_src.data(), flag_src.size());
  }
  return ST_OK;
}

int st_layout_csr(const st_layout* lay, int kind, int32_t* row_ptr, size_t row_ptr_cap, int32_t* col_idx,
                  size_t col_idx_cap, uint8_t* flags, size_t flags_cap) {
  const KindLayout* L = kind_of(lay, kind, "st_layout_csr");
  if (!L) return ST_ERR_INVALID;
  return copy_sparse("st_layout_csr", L->row_ptr, L->col_idx, L->flags, row_ptr, row_ptr_cap, col_idx, col_idx_cap,
                     flags, flags_cap);
}

int st_layout_csc(const st_layout* lay, int kind, int32_t* col_ptr, size_t col_ptr_cap, int32_t* row_idx,
                  size_t row_idx_cap, uint8_t* flags, size_t flags_cap) {
  const KindLayout* L = kind_of(lay, kind, "st_layout_csc");
  if (!L) return ST_ERR_INVALID;
  return copy_sparse("st_layout_csc", L->col_ptr, L->row_idx, L->csc_flags, col_ptr, col_ptr_cap, row_idx,
                     row_idx_cap, flags, flags_cap);
}

void st_layout_free(st_layout* lay) { delete lay; }

int st_block_size(void) { return kBlock; }

const char* st_status_string(int status) {
  switch (status) {
    case ST_OK: return "ok";
    case ST_ERR_INVALID: return "invalid argument";
    case ST_ERR_UNSUPPORTED: return "unsupported configuration";
    case ST_ERR_HIP: return "HIP runtime error";
    case ST_ERR_NOMEM: return "out of memory";
    case ST_ERR_BUFFER_TOO_SMALL: return "caller buffer too small";
    default: return "unknown status";
  }
}

const char* st_last_error(void) { return last_error_cstr(); }

}  // extern "C"
