// Kernel argument blocks and launchers (host <-> device interface of libst).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "st.h"
#include "st_device.hpp"

namespace st {

// Calls f(c0, c1, m) with the kind codes of `pattern`'s two head kinds and
// whether its heads are merged (two passes) as std::integral_constant values,
// so that launchers can pick kernels specialised on them.
template <class F>
hipError_t with_kind_codes(int pattern, F&& f) {
  using std::integral_constant;
  using plain = integral_constant<bool, false>;
  using merged = integral_constant<bool, true>;
  switch (pattern) {
    case ST_STRIDED: return f(integral_constant<int, K_LOCAL>(), integral_constant<int, K_STRIDE>(), plain());
    case ST_FIXED: return f(integral_constant<int, K_BLOCK>(), integral_constant<int, K_SUMMARY>(), plain());
    case ST_FIXED_R1: return f(integral_constant<int, K_BLOCK>(), integral_constant<int, K_SUMMARY_R1>(), plain());
    case ST_STRIDED_UNION:
      return f(integral_constant<int, K_LOCAL>(), integral_constant<int, K_STRIDE_X>(), merged());
    case ST_FIXED_UNION: return f(integral_constant<int, K_BLOCK>(), integral_constant<int, K_SUMMARY>(), merged());
    default: return f(integral_constant<int, K_CAUSAL>(), integral_constant<int, K_CAUSAL>(), plain());
  }
}

// True for the merged-head patterns (two passes over every head).
inline bool is_union(int pattern) { return pattern == ST_STRIDED_UNION || pattern == ST_FIXED_UNION; }

// Where a launch stores its results.  A plain head writes them (OUT_FINAL).
// A merged head runs two passes over the same rows and keys: the first
// (OUT_CARRY) keeps its fp32 results in the carry buffers, except for keys the
// second pass never holds, which it finishes itself; the second (OUT_MERGE)
// combines its own results with the carried ones and writes the outputs.
enum OutMode : int { OUT_FINAL = 0, OUT_CARRY = 1, OUT_MERGE = 2 };

// Work item of the dK/dV pass: key block kb of head bh, CSC entries [e0, e1).
// slot >= 0: the key block is split over several items and this one writes
// fp32 partial sums to workspace slot `slot`; slot < 0: write dk / dv directly.
// bf16: entries [e0, e_lo) are row blocks whose weights and dS enter dV and dK
// with their low parts too.
struct DkdvItem {
  int kb, bh, e0, e1, slot, kind, e_lo, pad;
};

// Work item of the forward and dq passes: row block qb of head bh, whose
// head kind (0 or 1) is `kind`.
struct RowItem {
  int qb, bh, kind, pad;
};

// Work item of the 16-bit forward and dq passes: the pair of 64-row LUT blocks
// 2pb and 2pb+1 of head bh (head kind `kind`).  Its key-block list is the
// kind's pair_entry[e0, e1); `first` repeats pair_entry[e0] (when e0 < e1) so
// that the first tile load is issued without reading the list.
// `flags`: kPairLo when a row of the pair attends at most kDqLoKeys keys (the
// dq pass then takes such rows' Delta exactly and carries dS to dQ as hi + lo),
// kPairPre when such a row's exact Delta comes from the delta pre-pass.
struct PairItem {
  int pb, bh, kind, e0, e1;
  uint32_t first;
  int flags, pad;
};
constexpr int kPairLo = 1, kPairPre = 2;

// Rows (per position, per head kind) that attend at most kDqLoKeys keys
// (merged heads: both passes together).  Their bf16 weights and dS are large,
// so the dq pass gives them an exact Delta and dS as hi + lo.  ROW_INBLOCK:
// the row's keys lie in one 64-key block, so the dq pass computes its exact
// Delta inside that block; ROW_PRE: the delta pre-pass computes it.
// ROW_NOKEY: the position is no key of the kind (nobody attends it, so its dk
// and dv are zero); the dq pass of a summary kind with an explicit summary set
// reads it instead of searching the set.
constexpr int kDqLoKeys = 32;
enum RowFlag : uint8_t { ROW_LO = 1, ROW_INBLOCK = 2, ROW_PRE = 4, ROW_NOKEY = 8 };

// Reduction of a split key block: partial slots [slot0, slot0 + nsplit).
struct ReduceItem {
  int kb, bh, slot0, nsplit, kind, pad0, pad1, pad2;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int H, T;
  const KindDev* kinds;  // [2], device memory
  const RowItem* items;  // fp32 kernel: row blocks
  const PairItem* pairs;  // 16-bit kernel: row-block pairs
  float sl2;             // log2(e) / sqrt(D)
  int pattern;           // ST_* (host side: selects the kernel)
  int out_mode;          // OutMode
  float* carry_o;        // merged heads: [B*H*T*D] first-pass output (fp32)
  float* carry_lse;      // merged heads: [B*H*T] first-pass lse, log2 units
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* ndelta;   // [B*H*T] workspace, fp32 path: -Delta for the dq and dk/dv passes
  float* ndelta_pre;  // [B*H*T] workspace: -Delta of ROW_PRE rows, from the delta pre-pass
  float* rowvals;  // [B*H*T][2] workspace, 16-bit path: lse * log2(e) and -Delta (exact) of each row, from dq
  float* partial;  // [slots][2][64][D] workspace: split dK / dV sums
  int BH, H, T;
  const KindDev* kinds;
  const RowItem* dq_items;   // fp32 dq: row blocks
  const PairItem* dq_pairs;  // 16-bit dq: row-block pairs
  const DkdvItem* dkdv_items;
  const ReduceItem* red_items;
  float sl2;    // log2(e) / sqrt(D)
  float scale;  // 1 / sqrt(D)
  int pattern;  // ST_* (host side: selects the kernels)
  int out_mode;  // OutMode
  float* carry_dq;  // merged heads: [B*H*T*D] first-pass gradients (fp32)
  float* carry_dk;
  float* carry_dv;
};

// Kernel ids for the optional launch timing (names in kKernelNames).
enum KernelId : int { KID_FWD = 0, KID_PRE, KID_DQ, KID_DKDV, KID_RED, KID_DELTA, KID_COUNT };
extern const char* const kKernelNames[KID_COUNT];

// Record timing events around a launch when timing is enabled (no-op otherwise).
void timing_begin(int kid, hipStream_t stream);
void timing_end(int kid, hipStream_t stream);

// rows_per_wave: 16 selects the eight-wave forward (16-bit inputs, D <= 64
// only); any other value, and every other case, the four-wave one (32 rows per
// wave).
template <typename TE, int D>
hipError_t launch_fwd(const FwdArgs& a, int n_items, int rows_per_wave, hipStream_t stream);

// The backward in two stages: Delta (fp32) and dq, then dk / dv and the
// reduction of split key blocks, which read the Delta the first stage wrote.
template <typename TE, int D>
hipError_t launch_bwd_delta(const BwdArgs& a, int n_items, hipStream_t stream);  // 16-bit only
template <typename TE, int D>
hipError_t launch_bwd_dq(const BwdArgs& a, int n_dq, hipStream_t stream);
// keys_per_wave: 32 selects the two-tile dk/dv kernel (16-bit inputs, D <= 64
// only); any other value, and every other case, the one-tile kernel.
template <typename TE, int D>
hipError_t launch_bwd_dkdv(const BwdArgs& a, int n_dkdv, int n_red, int keys_per_wave, hipStream_t stream);

}  // namespace st
