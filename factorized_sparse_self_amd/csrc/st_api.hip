// C ABI of libst: argument checks, the per-device plan cache (block LUTs of
// both head kinds plus the work schedules), the backward workspace, and the
// kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>
#include <map>
#include <set>
#include <memory>
#include <mutex>
#include <string>
#include <tuple>
#include <type_traits>
#include <vector>

#include "../../include/st.h"
#include "st_internal.hpp"
#include "st_kernels.hpp"

namespace st {

namespace {

// A key block of the dK/dV pass is split (fp32 partials, summed by the reduce
// kernel) only where its row-block list would outlast the launch: lists longer
// than half the average load of kDkdvSlots resident workgroups, and never into
// pieces shorter than kDkdvSplit row blocks.  Short launches with long columns
// (summary heads) split at kDkdvSplit; launches with many more items than the
// GPU holds (full attention, long sequences) are balanced by the schedule alone
// and split nothing, which spares the partials' workspace and traffic.
constexpr int kDkdvSplit = 24;
constexpr int64_t kDkdvSlots = 2048;

// Keys per wave of the 16-bit dK/dV kernel: 0 = by launch (32 for launches
// whose items far outnumber the GPU's slots, 16 otherwise), or 16 / 32 for
// every launch (st_set_dkdv_keys_per_wave).
std::atomic<int> g_dkdv_keys_per_wave{0};

// Rows per wave of the 16-bit forward: 0 = by launch (16, the eight-wave
// form, for launches of at most kFwdShortItems pair items, 32 otherwise), or
// 16 / 32 for every launch (st_set_fwd_rows_per_wave).  kFwdShortItems is one
// and a half rounds of the four-wave form on MI355X (256 CUs x 4 workgroups):
// at that size or less the eight-wave form, three workgroups per CU, hides
// more of each item's latency than it loses to its extra LDS reads.
constexpr int kFwdShortItems = 1536;
std::atomic<int> g_fwd_rows_per_wave{0};

struct PlanKey {
  int device, pattern, T, l, c, B, H;
  std::vector<int32_t> summary;  // canonical summary set (empty: the last c offsets)
  bool operator<(const PlanKey& o) const {
    return std::tie(device, pattern, T, l, c, B, H, summary) <
           std::tie(o.device, o.pattern, o.T, o.l, o.c, o.B, o.H, o.summary);
  }
};

// Work items of one pass over the heads.  A plain pattern runs one pass in
// which each head has its own kind; a merged head runs pass p over every head
// with kind p.
struct PassItems {
  RowItem* row_items = nullptr;    // row blocks: fp32 forward and dq
  PairItem* pair_items = nullptr;  // row-block pairs: 16-bit forward and dq
  PairItem* pre_items = nullptr;   // the pairs with kPairPre: 16-bit delta pre-pass
  DkdvItem* dkdv_items = nullptr;
  ReduceItem* red_items = nullptr;
  int n_row_items = 0, n_pair_items = 0, n_pre_items = 0, n_dkdv_items = 0, n_red_items = 0;
  bool dkdv_long = false;  // dK/dV items far outnumber the GPU's slots (no key block split)
};

struct Plan {
  void* dmem = nullptr;  // single device allocation holding everything below
  KindDev* kinds = nullptr;
  int n_pass = 1;
  PassItems pass[2];
  int n_slots = 0;  // partial slots of the dK/dV split (passes reuse them)
  ~Plan() {
    if (dmem) (void)hipFree(dmem);
  }
};

// Per-device workspace.  Calls on different streams are ordered on it: each
// call that uses it records `done` on its stream, and a call on another stream
// first makes its stream wait for that event.  The event only orders kernels
// of one device (every kernel ends with a device-wide release of its writes),
// so it is recorded without the system-scope fence, which would write the
// caches back for the host on every call (about 1.5 us between the kernels of
// consecutive steps).
struct Workspace {
  void* p = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;
  hipStream_t stream = nullptr;  // stream of the last call that used it
  bool used = false;
};

// At most kMaxPlans cached plans (per process); past that the least recently
// used one is dropped, after its device has finished every queued kernel.
constexpr size_t kMaxPlans = 64;

std::mutex g_mutex;
std::map<PlanKey, std::unique_ptr<Plan>> g_plans;
std::map<PlanKey, uint64_t> g_plan_use;  // last use (a counter) of each cached plan
uint64_t g_plan_clock = 0;
std::map<int, Workspace> g_workspace;

int hip_fail(const char* what, hipError_t e) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return ST_ERR_HIP;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Host image of a plan: byte blob plus the offsets of its parts.
struct Blob {
  std::vector<unsigned char> bytes;
  size_t add(const void* src, size_t n) {
    const size_t off = align_up(bytes.size(), 256);
    bytes.resize(off + std::max<size_t>(n, 1));
    if (n) std::memcpy(bytes.data() + off, src, n);
    return off;
  }
};

// Workgroup i of a launch is dispatched to XCD (i mod kXcds); each XCD has its
// own L2.  Items are grouped by the inputs they share, groups are assigned to
// XCDs longest-first (balancing total cost), each XCD's queue runs longest
// first, and queue x fills workgroup ids x, x + kXcds, ...  Short queues are
// padded with -1 (an empty item).  Items that cost at most `short_cost` count
// as equally long and keep their input order, so that short neighbours which
// read the same blocks (adjacent key blocks of a window or of an l-block in
// dk/dv) run at the same time and share the XCD's L2, instead of being
// separated by a sort on their small cost differences.
constexpr int kXcds = 8;
// Aim for at least this many groups so that every XCD gets several.
constexpr int kMinGroups = 64;

std::vector<int> xcd_order(const std::vector<int64_t>& cost, const std::vector<int64_t>& group,
                           int64_t short_cost = 0) {
  const size_t n = cost.size();
  std::map<int64_t, int64_t> gcost;
  for (size_t i = 0; i < n; ++i) gcost[group[i]] += cost[i];
  std::vector<std::pair<int64_t, int64_t>> gs(gcost.begin(), gcost.end());  // (group, cost)
  std::stable_sort(gs.begin(), gs.end(), [](const auto& x, const auto& y) { return x.second > y.second; });
  std::map<int64_t, int> gxcd;
  int64_t load[kXcds] = {};
  for (const auto& gc : gs) {
    const int x = (int)(std::min_element(load, load + kXcds) - load);
    gxcd[gc.first] = x;
    load[x] += gc.second;
  }
  std::vector<std::vector<int>> q(kXcds);
  for (size_t i = 0; i < n; ++i) q[gxcd[group[i]]].push_back((int)i);
  size_t maxlen = 0;
  for (auto& v : q) {
    std::stable_sort(v.begin(), v.end(),
                     [&](int x, int y) { return std::max(cost[x], short_cost) > std::max(cost[y], short_cost); });
    maxlen = std::max(maxlen, v.size());
  }
  std::vector<int> order(kXcds * maxlen, -1);
  for (int x = 0; x < kXcds; ++x)
    for (size_t j = 0; j < q[x].size(); ++j) order[j * kXcds + x] = q[x][j];
  return order;
}

int build_plan(const PlanKey& key, Plan* plan) {
  st_layout lay;
  lay.pattern = key.pattern;
  lay.T = key.T;
  lay.l = key.l;
  lay.c = key.c;
  lay.summary = key.summary;
  const int32_t* sigma_host = lay.summary.empty() ? nullptr : lay.summary.data();
  for (int kind = 0; kind < 2; ++kind) {
    make_geometry(key.pattern, kind, key.T, key.l, key.c, sigma_host, &lay.kind[kind].geo);
    build_kind(lay.kind[kind]);
  }
  const int BH = key.B * key.H;
  const int chunks_per_head = std::max(1, (kMinGroups + BH - 1) / BH);
  int chunk[2];
  for (int kind = 0; kind < 2; ++kind)
    chunk[kind] = std::max(1, (lay.kind[kind].n_qb + chunks_per_head - 1) / chunks_per_head);

  // Row-block pairs: the CSR rows of blocks 2p and 2p+1 merged (both ascending)
  // into one list of key blocks with per-half visit / FULL bits.
  std::vector<int32_t> pair_ptr[2];
  std::vector<uint32_t> pair_entry[2];
  for (int kind = 0; kind < 2; ++kind) {
    const KindLayout& L = lay.kind[kind];
    const int n_pairs = (L.n_qb + 1) / 2;
    pair_ptr[kind].assign(n_pairs + 1, 0);
    for (int pb = 0; pb < n_pairs; ++pb) {
      int i0 = L.row_ptr[2 * pb], e0 = L.row_ptr[2 * pb + 1];
      int i1 = 2 * pb + 1 < L.n_qb ? L.row_ptr[2 * pb + 1] : 0, e1 = 2 * pb + 1 < L.n_qb ? L.row_ptr[2 * pb + 2] : 0;
      while (i0 < e0 || i1 < e1) {
        const int k0 = i0 < e0 ? L.col_idx[i0] : INT_MAX, k1 = i1 < e1 ? L.col_idx[i1] : INT_MAX;
        const int kb = std::min(k0, k1);
        uint32_t bits = (uint32_t)kb;
        if (k0 == kb) bits |= (kPairVisit | (L.flags[i0++] ? kPairFull : 0u)) << 28;
        if (k1 == kb) bits |= (kPairVisit | (L.flags[i1++] ? kPairFull : 0u)) << 30;
        pair_entry[kind].push_back(bits);
      }
      pair_ptr[kind][pb + 1] = (int32_t)pair_entry[kind].size();
    }
  }
  // Row blocks whose weights and dS enter the bf16 dV and dK products with
  // their low parts too: those with a row that attends at most n_lo keys.  A
  // row with n keys gives each weights of about 1/n, and the bf16 rounding
  // errors of the weights a key receives walk randomly, with a variance
  // proportional to the sum of their squares.  Where each row adds one key to
  // the next (window, strided, own-block and full attention) the rows past
  // n_lo = 64 keys add about e/n_lo to that sum (e for the spread of softmax
  // weights under Gaussian logits); a summary row in l-block b attends c*b
  // keys and l rows share that count, so rows past K blocks add about
  // e l / (c^2 K), and K = ceil(8 l / c^2) keeps it at about 1/3 too.
  auto lo_keys = [&](const Geometry& g) -> int64_t {
    if (g.code != K_SUMMARY && g.code != K_SUMMARY_R1) return 64;
    const int64_t cc = std::max(1, g.c);
    return std::max<int64_t>(64, cc * ((8 * (int64_t)g.l + cc * cc - 1) / (cc * cc)));
  };
  std::vector<uint8_t> lo_block[2];
  for (int kind = 0; kind < 2; ++kind) {
    const KindLayout& L = lay.kind[kind];
    const int64_t n_lo = lo_keys(L.geo);
    lo_block[kind].assign(L.n_qb, 0);
    for (int qb = 0; qb < L.n_qb; ++qb)
      for (int i = 0; i < kBlock; ++i) {
        const int R = qb * kBlock + i;
        const int t = row_position(L.geo, R);
        if (t < 0) continue;
        int lo = 1, hi = 0;
        row_interval(L.geo, R, t, lo, hi);
        if (lo <= hi && hi - lo + 1 <= n_lo) {
          lo_block[kind][qb] = 1;
          break;
        }
      }
  }
  // first CSC entry in [a, b) whose row block needs no low part (along a key
  // block's list the rows' key counts only grow, so the others precede it)
  auto entry_lo = [&](int kind, int a, int b) {
    const KindLayout& L = lay.kind[kind];
    while (a < b && lo_block[kind][L.row_idx[a]]) ++a;
    return a;
  };
  const bool merged = is_union(key.pattern);
  const int n_pass = merged ? 2 : 1;
  // Per position: the keys each kind gives it, whether they lie in one 64-key
  // block, and from these the RowFlag bits of the 16-bit dq (a merged head
  // counts both kinds' keys; its Delta always comes from the pre-pass, since
  // each dq pass sees only one kind's keys).
  std::vector<int32_t> n_keys[2];
  std::vector<uint8_t> one_block[2], row_flags[2];
  for (int kind = 0; kind < 2; ++kind) {
    const KindLayout& L = lay.kind[kind];
    n_keys[kind].assign(key.T, 0);
    one_block[kind].assign(key.T, 0);
    for (int R = 0; R < L.geo.n_rows; ++R) {
      const int t = row_position(L.geo, R);
      if (t < 0) continue;
      int lo = 1, hi = 0;
      row_interval(L.geo, R, t, lo, hi);
      if (lo > hi) continue;
      n_keys[kind][t] = hi - lo + 1;
      one_block[kind][t] = lo / kBlock == hi / kBlock;
    }
  }
  for (int kind = 0; kind < 2; ++kind) {
    row_flags[kind].assign(key.T, 0);
    for (int t = 0; t < key.T; ++t) {
      if (!position_is_key(lay.kind[kind].geo, t)) row_flags[kind][t] = ROW_NOKEY;
      const int n = merged ? n_keys[0][t] + n_keys[1][t] : n_keys[kind][t];
      if (n == 0 || n > kDqLoKeys) continue;
      uint8_t f = ROW_LO;
      if (!merged && one_block[kind][t])
        f |= ROW_INBLOCK;
      else
        f |= ROW_PRE;
      row_flags[kind][t] |= f;
    }
  }
  // kPairLo / kPairPre of the pair of row blocks (2pb, 2pb+1) of a kind: rows
  // that attend keys of that kind only count
  auto pair_flags = [&](int kind, int pb) {
    const KindLayout& L = lay.kind[kind];
    int f = 0;
    for (int R = 2 * pb * kBlock; R < std::min(L.geo.n_rows, (2 * pb + 2) * kBlock); ++R) {
      const int t = row_position(L.geo, R);
      if (t < 0 || n_keys[kind][t] == 0) continue;
      if (row_flags[kind][t] & ROW_LO) f |= kPairLo;
      if (row_flags[kind][t] & ROW_PRE) f |= kPairPre;
    }
    return f;
  };
  std::vector<int> pflags[2];
  for (int kind = 0; kind < 2; ++kind) {
    const int n_pairs = (int)pair_ptr[kind].size() - 1;
    pflags[kind].resize(n_pairs);
    for (int pb = 0; pb < n_pairs; ++pb) pflags[kind][pb] = pair_flags(kind, pb);
  }
  // kind of head bh in pass p
  auto kind_of = [&](int p, int bh) { return merged ? p : (bh % key.H) & 1; };
  struct HostPass {
    std::vector<RowItem> rows;
    std::vector<PairItem> pairs, pre;
    std::vector<DkdvItem> dkdv;
    std::vector<ReduceItem> red;
    bool dkdv_long = false;
  } hp[2];
  int max_slots = 0;
  for (int p = 0; p < n_pass; ++p) {
    // Row-block items (fp32 forward, dq): every row block of every head; cost
    // = key blocks visited + 1; grouped by (head, range of row blocks).
    std::vector<RowItem> rows;
    std::vector<int64_t> rcost, rgroup;
    for (int bh = 0; bh < BH; ++bh) {
      const int kind = kind_of(p, bh);
      const KindLayout& L = lay.kind[kind];
      for (int qb = 0; qb < L.n_qb; ++qb) {
        rows.push_back({qb, bh, kind, 0});
        rcost.push_back(L.row_ptr[qb + 1] - L.row_ptr[qb] + 1);
        rgroup.push_back((int64_t)bh * 65536 + qb / chunk[kind]);
      }
    }
    for (int i : xcd_order(rcost, rgroup)) hp[p].rows.push_back(i < 0 ? RowItem{-1, -1, 0, 0} : rows[i]);

    // Row-block pair items (16-bit forward and dq).
    std::vector<PairItem> pairs;
    std::vector<int64_t> pcost, pgroup;
    for (int bh = 0; bh < BH; ++bh) {
      const int kind = kind_of(p, bh);
      const int n_pairs = (int)pair_ptr[kind].size() - 1;
      for (int pb = 0; pb < n_pairs; ++pb) {
        const int e0 = pair_ptr[kind][pb], e1 = pair_ptr[kind][pb + 1];
        pairs.push_back({pb, bh, kind, e0, e1, e1 > e0 ? pair_entry[kind][e0] : 0u, pflags[kind][pb], 0});
        pcost.push_back(e1 - e0 + 1);
        pgroup.push_back((int64_t)bh * 65536 + 2 * pb / chunk[kind]);
      }
    }
    for (int i : xcd_order(pcost, pgroup))
      hp[p].pairs.push_back(i < 0 ? PairItem{-1, -1, 0, 0, 0, 0u, 0, 0} : pairs[i]);
    // the delta pre-pass: pairs that hold a ROW_PRE row
    {
      std::vector<PairItem> pre;
      std::vector<int64_t> cost, group;
      for (const PairItem& it : pairs)
        if (it.flags & kPairPre) {
          pre.push_back(it);
          cost.push_back(it.e1 - it.e0 + 1);
          group.push_back((int64_t)it.bh * 65536 + 2 * it.pb / chunk[it.kind]);
        }
      if (!pre.empty())
        for (int i : xcd_order(cost, group))
          hp[p].pre.push_back(i < 0 ? PairItem{-1, -1, 0, 0, 0, 0u, 0, 0} : pre[i]);
    }

    // dK/dV items: every key block of every head.  A key block whose row-block
    // list is longer than `split` is split at row-block multiples of `split`,
    // so that the splits of different key blocks read the same row blocks;
    // grouped by (head, first row block read).
    int64_t dwork = 0;
    for (int bh = 0; bh < BH; ++bh) {
      const KindLayout& L = lay.kind[kind_of(p, bh)];
      dwork += L.col_ptr[L.n_kb] + L.n_kb;
    }
    const int64_t avg = (dwork + kDkdvSlots - 1) / kDkdvSlots;
    const int64_t avg_up = (avg + kDkdvSplit - 1) / kDkdvSplit * kDkdvSplit;  // a multiple of kDkdvSplit
    const int split = (int)std::min<int64_t>(std::max<int64_t>(kDkdvSplit, avg_up), 1 << 30);
    hp[p].dkdv_long = split > kDkdvSplit;
    std::vector<DkdvItem> dkdv;
    std::vector<int64_t> dcost, dgroup;
    int slots = 0;
    for (int bh = 0; bh < BH; ++bh) {
      const int kind = kind_of(p, bh);
      const KindLayout& L = lay.kind[kind];
      for (int kb = 0; kb < L.n_kb; ++kb) {
        const int e0 = L.col_ptr[kb], e1 = L.col_ptr[kb + 1];
        const int first_q = e1 > e0 ? L.row_idx[e0] : 0;
        if (e1 - e0 <= split) {
          dkdv.push_back({kb, bh, e0, e1, -1, kind, entry_lo(kind, e0, e1), 0});
          dcost.push_back(e1 - e0 + 1);
          dgroup.push_back((int64_t)bh * 65536 + first_q / chunk[kind]);
          continue;
        }
        const int slot0 = slots;
        for (int a = e0; a < e1;) {
          const int range = L.row_idx[a] / split;
          int b = a;
          while (b < e1 && L.row_idx[b] / split == range) ++b;
          dkdv.push_back({kb, bh, a, b, slots++, kind, entry_lo(kind, a, b), 0});
          dcost.push_back(b - a + 1);
          dgroup.push_back((int64_t)bh * 65536 + L.row_idx[a] / chunk[kind]);
          a = b;
        }
        hp[p].red.push_back({kb, bh, slot0, slots - slot0, kind, 0, 0, 0});
      }
    }
    // (an item's cost is its row-block count + 1; up to 4 the order is the
    // key-block order)
    for (int i : xcd_order(dcost, dgroup, 4))
      hp[p].dkdv.push_back(i < 0 ? DkdvItem{-1, -1, 0, 0, -1, 0, 0, 0} : dkdv[i]);
    max_slots = std::max(max_slots, slots);
  }
  Blob blob;
  KindDev kinds_host[2];
  size_t off_kinds = blob.add(kinds_host, sizeof(kinds_host));
  const size_t off_sigma = blob.add(lay.summary.data(), lay.summary.size() * sizeof(int32_t));
  size_t offs[2][11];
  for (int kind = 0; kind < 2; ++kind) {
    const KindLayout& L = lay.kind[kind];
    offs[kind][0] = blob.add(L.row_ptr.data(), L.row_ptr.size() * 4);
    offs[kind][1] = blob.add(L.col_idx.data(), L.col_idx.size() * 4);
    offs[kind][2] = blob.add(L.flags.data(), L.flags.size());
    offs[kind][3] = blob.add(L.col_ptr.data(), L.col_ptr.size() * 4);
    offs[kind][4] = blob.add(L.row_idx.data(), L.row_idx.size() * 4);
    offs[kind][5] = blob.add(L.csc_flags.data(), L.csc_flags.size());
    std::vector<uint32_t> csr(L.col_idx.size()), csc(L.row_idx.size());
    for (size_t e = 0; e < csr.size(); ++e) csr[e] = (uint32_t)L.col_idx[e] | (L.flags[e] ? kFullBit : 0u);
    for (size_t e = 0; e < csc.size(); ++e) csc[e] = (uint32_t)L.row_idx[e] | (L.csc_flags[e] ? kFullBit : 0u);
    offs[kind][6] = blob.add(csr.data(), csr.size() * 4);
    offs[kind][7] = blob.add(csc.data(), csc.size() * 4);
    offs[kind][8] = blob.add(pair_ptr[kind].data(), pair_ptr[kind].size() * 4);
    offs[kind][9] = blob.add(pair_entry[kind].data(), pair_entry[kind].size() * 4);
    offs[kind][10] = blob.add(row_flags[kind].data(), row_flags[kind].size());
  }
  size_t off_items[2][5];
  for (int p = 0; p < n_pass; ++p) {
    off_items[p][0] = blob.add(hp[p].rows.data(), hp[p].rows.size() * sizeof(RowItem));
    off_items[p][1] = blob.add(hp[p].pairs.data(), hp[p].pairs.size() * sizeof(PairItem));
    off_items[p][4] = blob.add(hp[p].pre.data(), hp[p].pre.size() * sizeof(PairItem));
    off_items[p][2] = blob.add(hp[p].dkdv.data(), hp[p].dkdv.size() * sizeof(DkdvItem));
    off_items[p][3] = blob.add(hp[p].red.data(), hp[p].red.size() * sizeof(ReduceItem));
  }

  hipError_t e = hipMalloc(&plan->dmem, blob.bytes.size());
  if (e != hipSuccess) {
    plan->dmem = nullptr;
    set_error(std::string("plan allocation: ") + hipGetErrorString(e));
    return ST_ERR_NOMEM;
  }
  unsigned char* dbase = (unsigned char*)plan->dmem;
  for (int kind = 0; kind < 2; ++kind) {
    const KindLayout& L = lay.kind[kind];
    KindDev& k = kinds_host[kind];
    k.geo = L.geo;
    k.geo.sigma = lay.summary.empty() ? nullptr : (const int32_t*)(dbase + off_sigma);
    k.row_ptr = (const int32_t*)(dbase + offs[kind][0]);
    k.col_idx = (const int32_t*)(dbase + offs[kind][1]);
    k.flags = (const uint8_t*)(dbase + offs[kind][2]);
    k.col_ptr = (const int32_t*)(dbase + offs[kind][3]);
    k.row_idx = (const int32_t*)(dbase + offs[kind][4]);
    k.csc_flags = (const uint8_t*)(dbase + offs[kind][5]);
    k.csr_entry = (const uint32_t*)(dbase + offs[kind][6]);
    k.csc_entry = (const uint32_t*)(dbase + offs[kind][7]);
    k.pair_ptr = (const int32_t*)(dbase + offs[kind][8]);
    k.pair_entry = (const uint32_t*)(dbase + offs[kind][9]);
    k.row_flags = (const uint8_t*)(dbase + offs[kind][10]);
  }
  std::memcpy(blob.bytes.data() + off_kinds, kinds_host, sizeof(kinds_host));
  e = hipMemcpy(plan->dmem, blob.bytes.data(), blob.bytes.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail("plan upload", e);
  plan->kinds = (KindDev*)(dbase + off_kinds);
  plan->n_pass = n_pass;
  for (int p = 0; p < n_pass; ++p) {
    PassItems& P = plan->pass[p];
    P.row_items = (RowItem*)(dbase + off_items[p][0]);
    P.pair_items = (PairItem*)(dbase + off_items[p][1]);
    P.pre_items = (PairItem*)(dbase + off_items[p][4]);
    P.dkdv_items = (DkdvItem*)(dbase + off_items[p][2]);
    P.red_items = (ReduceItem*)(dbase + off_items[p][3]);
    P.n_row_items = (int)hp[p].rows.size();
    P.n_pair_items = (int)hp[p].pairs.size();
    P.n_pre_items = (int)hp[p].pre.size();
    P.n_dkdv_items = (int)hp[p].dkdv.size();
    P.n_red_items = (int)hp[p].red.size();
    P.dkdv_long = hp[p].dkdv_long;
  }
  plan->n_slots = max_slots;
  return ST_OK;
}

// Caller holds g_mutex.  A cached plan, or (build == true) a new one.
int get_plan(const PlanKey& key, Plan** out, bool build = true) {
  auto it = g_plans.find(key);
  if (it != g_plans.end()) {
    g_plan_use[key] = ++g_plan_clock;
    *out = it->second.get();
    return ST_OK;
  }
  if (!build) {
    set_error("no cached plan for this shape and pattern: one call of another attention entry point with "
              "the same shapes builds it");
    return ST_ERR_UNSUPPORTED;
  }
  if (g_plans.size() >= kMaxPlans) {
    auto lru = std::min_element(g_plan_use.begin(), g_plan_use.end(),
                                [](const auto& x, const auto& y) { return x.second < y.second; });
    const PlanKey old = lru->first;
    int current = 0;
    if (hipGetDevice(&current) != hipSuccess) return hip_fail("plan cache", hipErrorInvalidDevice);
    // kernels still queued may read the plan: let its device drain first
    hipError_t e = hipSetDevice(old.device);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail("plan cache eviction", e);
    g_plans.erase(old);
    g_plan_use.erase(old);
    e = hipSetDevice(current);
    if (e != hipSuccess) return hip_fail("plan cache eviction", e);
  }
  std::unique_ptr<Plan> plan(new Plan);
  const int rc = build_plan(key, plan.get());
  if (rc != ST_OK) return rc;
  *out = plan.get();
  g_plans[key] = std::move(plan);
  g_plan_use[key] = ++g_plan_clock;
  return ST_OK;
}

// Caller holds g_mutex.  The device's workspace, at least `bytes` large, made
// safe for kernels on `stream`: if the last call that used it ran on another
// stream, `stream` first waits for that call's kernels.  Pair with
// workspace_done() once the call's kernels are queued.
int get_workspace(int device, size_t bytes, hipStream_t stream, void** out) {
  Workspace& w = g_workspace[device];
  hipError_t e = hipSuccess;
  if (!w.done) {
    e = hipEventCreateWithFlags(&w.done, hipEventDisableTiming | hipEventDisableSystemFence);
    if (e != hipSuccess) {
      w.done = nullptr;
      return hip_fail("workspace event", e);
    }
  }
  if (w.bytes < bytes) {
    // the old buffer may still be in use by queued kernels
    if (w.used) {
      e = hipEventSynchronize(w.done);
      if (e != hipSuccess) return hip_fail("workspace", e);
    }
    if (w.p) (void)hipFree(w.p);
    w.p = nullptr;
    w.bytes = 0;
    e = hipMalloc(&w.p, bytes);
    if (e != hipSuccess) {
      w.p = nullptr;
      set_error(std::string("workspace allocation: ") + hipGetErrorString(e));
      return ST_ERR_NOMEM;
    }
    w.bytes = bytes;
  } else if (w.used && w.stream != stream) {
    e = hipStreamWaitEvent(stream, w.done, 0);
    if (e != hipSuccess) return hip_fail("workspace", e);
  }
  *out = w.p;
  return ST_OK;
}

// Caller holds g_mutex: the call's kernels that use the workspace are queued on `stream`.
int workspace_done(int device, hipStream_t stream) {
  Workspace& w = g_workspace[device];
  const hipError_t e = hipEventRecord(w.done, stream);
  if (e != hipSuccess) return hip_fail("workspace", e);
  w.stream = stream;
  w.used = true;
  return ST_OK;
}

// The static scratch of st_sparse_attn_bwd_noalloc: one copy per device, held
// until the process ends.  Host code never uses the symbol itself as an
// address: scratch_address() returns this device's copy, looked up once per
// device with hipGetSymbolAddress.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::map<int, void*> g_scratch;  // device -> address of its copy

// Caller holds g_mutex; `device` is current.
int scratch_address(int device, void** out) {
  auto it = g_scratch.find(device);
  if (it == g_scratch.end()) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail("static scratch address", e != hipSuccess ? e : hipErrorUnknown);
    it = g_scratch.emplace(device, ptr).first;
  }
  *out = it->second;
  return ST_OK;
}

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

int check_attn_args(const char* fn, const void* const* ptrs, int n_ptrs, int B, int H, int T, int D,
                    int pattern, int l, int c, const int32_t* summary) {
  for (int i = 0; i < n_ptrs; ++i)
    if (!aligned16(ptrs[i])) {
      set_error(std::string(fn) + ": tensor pointer " + std::to_string(i) +
                " is null or not 16-byte aligned");
      return ST_ERR_INVALID;
    }
  if (B < 1 || H < 1 || (int64_t)B * H > (1 << 20)) {
    set_error(std::string(fn) + ": need B >= 1, H >= 1, B*H <= 2^20");
    return ST_ERR_INVALID;
  }
  const std::string why = check_pattern_args(pattern, T, l, c, summary);
  if (!why.empty()) {
    set_error(std::string(fn) + ": " + why);
    return ST_ERR_INVALID;
  }
  if (D != 32 && D != 64 && D != 128) {
    set_error(std::string(fn) + ": head dimension D must be 32, 64 or 128, got " + std::to_string(D));
    return ST_ERR_UNSUPPORTED;
  }
  Geometry g;
  make_geometry(pattern, 1, T, l, c, nullptr, &g);
  const int64_t blocks = ((int64_t)std::max(g.n_rows, T) + kBlock - 1) / kBlock;
  if (blocks * B * H >= (int64_t)1 << 31) {
    set_error(std::string(fn) + ": too many work items for one launch");
    return ST_ERR_UNSUPPORTED;
  }
  return ST_OK;
}

// The 16-bit kernels address one head of a tensor through 32-bit buffer
// offsets: T*D*2 <= 2^31.
int check_head_size(const char* fn, bool path16, int T, int D) {
  if (path16 && (int64_t)T * D * 2 > ((int64_t)1 << 31)) {
    set_error(std::string(fn) + ": one head of a 16-bit tensor must fit in 2^31 bytes (T*D <= 2^30), got T=" +
              std::to_string(T) + ", D=" + std::to_string(D));
    return ST_ERR_UNSUPPORTED;
  }
  return ST_OK;
}

template <typename TE>
int attn_fwd(const char* fn, const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int H, int T, int D, int pattern, int l, int c, const int32_t* summary, void* stream) {
  const void* ptrs[] = {q, k, v, out, lse};
  int rc = check_attn_args(fn, ptrs, 5, B, H, T, D, pattern, l, c, summary);
  if (rc != ST_OK) return rc;
  constexpr bool k16 = Is16<TE>::value;
  rc = check_head_size(fn, k16, T, D);
  if (rc != ST_OK) return rc;
  if (!uses_summary(pattern)) c = 0;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(fn, e);
  std::lock_guard<std::mutex> lock(g_mutex);
  Plan* plan = nullptr;
  rc = get_plan({device, pattern, T, l, c, B, H, canonical_summary(pattern, l, c, summary)}, &plan);
  if (rc != ST_OK) return rc;
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.lse = lse;
  a.H = H;
  a.T = T;
  a.kinds = plan->kinds;
  a.sl2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  a.pattern = pattern;
  a.out_mode = OUT_FINAL;
  a.carry_o = nullptr;
  a.carry_lse = nullptr;
  if (plan->n_pass == 2) {
    // first pass: fp32 output and lse of every row, merged by the second
    const size_t rows = (size_t)B * H * T;
    const size_t o_bytes = align_up(rows * D * sizeof(float), 256);
    void* ws = nullptr;
    rc = get_workspace(device, o_bytes + rows * sizeof(float), (hipStream_t)stream, &ws);
    if (rc != ST_OK) return rc;
    a.carry_o = (float*)ws;
    a.carry_lse = (float*)((unsigned char*)ws + o_bytes);
  }
  hipStream_t s = (hipStream_t)stream;
  for (int p = 0; p < plan->n_pass; ++p) {
    const PassItems& P = plan->pass[p];
    // 16-bit: one workgroup per pair of row blocks; fp32: per row block
    a.items = P.row_items;
    a.pairs = P.pair_items;
    const int n_items = k16 ? P.n_pair_items : P.n_row_items;
    if (plan->n_pass == 2) a.out_mode = p == 0 ? OUT_CARRY : OUT_MERGE;
    const int rpw_set = g_fwd_rows_per_wave.load(std::memory_order_relaxed);
    const int rpw = rpw_set ? rpw_set : n_items <= kFwdShortItems ? 16 : 32;
    e = D == 32 ? launch_fwd<TE, 32>(a, n_items, rpw, s)
        : D == 64 ? launch_fwd<TE, 64>(a, n_items, rpw, s)
                  : launch_fwd<TE, 128>(a, n_items, rpw, s);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  if (plan->n_pass == 2) return workspace_done(device, s);
  return ST_OK;
}

// Backward.  static_ws: the workspace is this device's static scratch and
// nothing is allocated (the plan must be cached already).
template <typename TE>
int attn_bwd(const char* fn, const void* q, const void* k, const void* v, const void* out,
             const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int H, int T,
             int D, int pattern, int l, int c, const int32_t* summary, void* stream, bool static_ws = false) {
  const void* ptrs[] = {q, k, v, out, lse, dout, dq, dk, dv};
  int rc = check_attn_args(fn, ptrs, 9, B, H, T, D, pattern, l, c, summary);
  if (rc != ST_OK) return rc;
  rc = check_head_size(fn, Is16<TE>::value, T, D);
  if (rc != ST_OK) return rc;
  if (!uses_summary(pattern)) c = 0;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(fn, e);
  std::lock_guard<std::mutex> lock(g_mutex);
  Plan* plan = nullptr;
  rc = get_plan({device, pattern, T, l, c, B, H, canonical_summary(pattern, l, c, summary)}, &plan, !static_ws);
  if (rc != ST_OK) return rc;
  // workspace: -Delta (fp32 path) or (lse2, -Delta) row pairs (16-bit path), split partials, for merged heads the first pass's
  // fp32 dq, dk, dv, and the pre-pass Delta
  const size_t rows = (size_t)B * H * T;
  const size_t delta_bytes = align_up(rows * sizeof(float), 256);
  const size_t partial_bytes = align_up((size_t)plan->n_slots * 2 * kBlock * D * sizeof(float), 256);
  const size_t carry_bytes = plan->n_pass == 2 ? align_up(rows * D * sizeof(float), 256) : 0;
  const size_t ws_bytes = 3 * delta_bytes + partial_bytes + 3 * carry_bytes;
  void* ws = nullptr;
  if (static_ws) {
    if (ws_bytes > kScratchBytes) {
      set_error(std::string(fn) + ": needs " + std::to_string(ws_bytes) + " bytes of scratch; the static scratch holds " +
                std::to_string(kScratchBytes));
      return ST_ERR_UNSUPPORTED;
    }
    rc = scratch_address(device, &ws);
  } else {
    rc = get_workspace(device, ws_bytes, (hipStream_t)stream, &ws);
  }
  if (rc != ST_OK) return rc;
  unsigned char* wb = (unsigned char*)ws;
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ndelta = (float*)wb;   // fp32 path
  a.rowvals = (float*)wb;  // 16-bit path: 8 bytes per row, the first two delta_bytes slots
  a.partial = (float*)(wb + 2 * delta_bytes);
  a.carry_dq = carry_bytes ? (float*)(wb + 2 * delta_bytes + partial_bytes) : nullptr;
  a.carry_dk = carry_bytes ? (float*)(wb + 2 * delta_bytes + partial_bytes + carry_bytes) : nullptr;
  a.carry_dv = carry_bytes ? (float*)(wb + 2 * delta_bytes + partial_bytes + 2 * carry_bytes) : nullptr;
  a.ndelta_pre = (float*)(wb + 2 * delta_bytes + partial_bytes + 3 * carry_bytes);
  a.BH = B * H;
  a.H = H;
  a.T = T;
  a.kinds = plan->kinds;
  a.scale = (float)(1.0 / std::sqrt((double)D));
  a.sl2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  a.pattern = pattern;
  a.out_mode = OUT_FINAL;
  hipStream_t s = (hipStream_t)stream;
  // Every dq launch precedes every dk/dv launch on the stream: the 16-bit dq
  // passes complete Delta, which dk/dv reads.  Merged heads: within each
  // stage the first pass (carry) precedes the second (merge).
  auto set_pass = [&](int p) {
    const PassItems& P = plan->pass[p];
    if (plan->n_pass == 2) a.out_mode = p == 0 ? OUT_CARRY : OUT_MERGE;
    // 16-bit dq: one workgroup per pair of row blocks; fp32: per row block
    a.dq_items = P.row_items;
    a.dq_pairs = P.pair_items;
    a.dkdv_items = P.dkdv_items;
    a.red_items = P.red_items;
  };
  // 16-bit: the delta pre-pass of every pass first (rows with few keys whose
  // exact Delta the dq pass cannot form inside one key block)
  if (Is16<TE>::value)
    for (int p = 0; p < plan->n_pass; ++p) {
      set_pass(p);
      const PassItems& P = plan->pass[p];
      if (P.n_pre_items == 0) continue;
      a.dq_pairs = P.pre_items;
      e = D == 32 ? launch_bwd_delta<TE, 32>(a, P.n_pre_items, s)
          : D == 64 ? launch_bwd_delta<TE, 64>(a, P.n_pre_items, s)
                    : launch_bwd_delta<TE, 128>(a, P.n_pre_items, s);
      if (e != hipSuccess) return hip_fail(fn, e);
    }
  for (int p = 0; p < plan->n_pass; ++p) {
    set_pass(p);
    const PassItems& P = plan->pass[p];
    const int n_dq = Is16<TE>::value ? P.n_pair_items : P.n_row_items;
    e = D == 32 ? launch_bwd_dq<TE, 32>(a, n_dq, s)
        : D == 64 ? launch_bwd_dq<TE, 64>(a, n_dq, s)
                  : launch_bwd_dq<TE, 128>(a, n_dq, s);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  const int kpw_set = g_dkdv_keys_per_wave.load(std::memory_order_relaxed);
  for (int p = 0; p < plan->n_pass; ++p) {
    set_pass(p);
    const PassItems& P = plan->pass[p];
    const int kpw = kpw_set ? kpw_set : P.dkdv_long ? 32 : 16;
    e = D == 32 ? launch_bwd_dkdv<TE, 32>(a, P.n_dkdv_items, P.n_red_items, kpw, s)
        : D == 64 ? launch_bwd_dkdv<TE, 64>(a, P.n_dkdv_items, P.n_red_items, kpw, s)
                  : launch_bwd_dkdv<TE, 128>(a, P.n_dkdv_items, P.n_red_items, kpw, s);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  return static_ws ? ST_OK : workspace_done(device, s);
}

// ---------------------------------------------------------------------------
// Launch timing: event pairs recorded around each launch while enabled.
// ---------------------------------------------------------------------------
struct TimingRecord {
  int kid;
  hipEvent_t start, stop;
};

std::mutex g_timing_mutex;
bool g_timing_on = false;
std::vector<TimingRecord> g_timing_records;
std::vector<hipEvent_t> g_event_pool;
TimingRecord g_open[KID_COUNT];
bool g_is_open[KID_COUNT] = {};
int64_t g_launches[KID_COUNT] = {};
double g_total_ms[KID_COUNT] = {};

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // timing only: no system-scope fence, whose cache write-back would lengthen
  // the kernels being timed
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Fold completed records into the per-kernel totals (caller holds the mutex).
int drain_records() {
  for (const TimingRecord& r : g_timing_records) {
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail("st_timing_read", e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail("st_timing_read", e);
    g_launches[r.kid] += 1;
    g_total_ms[r.kid] += ms;
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_timing_records.clear();
  return ST_OK;
}

}  // namespace

const char* const kKernelNames[KID_COUNT] = {"fwd", "bwd_pre", "bwd_dq", "bwd_dkdv", "bwd_reduce", "bwd_delta"};

void timing_begin(int kid, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_timing_mutex);
  g_is_open[kid] = false;
  if (!g_timing_on) return;
  TimingRecord r{kid, take_event(), take_event()};
  if (!r.start || !r.stop) return;
  if (hipEventRecord(r.start, stream) != hipSuccess) return;
  g_open[kid] = r;
  g_is_open[kid] = true;
}

void timing_end(int kid, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_timing_mutex);
  if (!g_is_open[kid]) return;
  g_is_open[kid] = false;
  if (hipEventRecord(g_open[kid].stop, stream) != hipSuccess) return;
  g_timing_records.push_back(g_open[kid]);
}

}  // namespace st

using namespace st;

extern "C" {

int st_sparse_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                       int H, int T, int D, int pattern, int l, int c, void* stream) {
  return attn_fwd<bf16>("st_sparse_attn_fwd", q, k, v, out, lse, B, H, T, D, pattern, l, c, nullptr, stream);
}

int st_sparse_attn_fwd_f16(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                           int H, int T, int D, int pattern, int l, int c, void* stream) {
  return attn_fwd<f16>("st_sparse_attn_fwd_f16", q, k, v, out, lse, B, H, T, D, pattern, l, c, nullptr, stream);
}

int st_sparse_attn_fwd_f32(const void* q, const void* k, const void* v, void* out, float* lse,
                           int B, int H, int T, int D, int pattern, int l, int c, void* stream) {
  return attn_fwd<float>("st_sparse_attn_fwd_f32", q, k, v, out, lse, B, H, T, D, pattern, l, c,
                         nullptr, stream);
}

int st_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                       int H, int T, int D, int pattern, int l, int c, void* stream) {
  return attn_bwd<bf16>("st_sparse_attn_bwd", q, k, v, out, lse, dout, dq, dk, dv, B, H, T, D,
                        pattern, l, c, nullptr, stream);
}

int st_sparse_attn_bwd_f16(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                           int H, int T, int D, int pattern, int l, int c, void* stream) {
  return attn_bwd<f16>("st_sparse_attn_bwd_f16", q, k, v, out, lse, dout, dq, dk, dv, B, H, T, D,
                       pattern, l, c, nullptr, stream);
}

int st_sparse_attn_bwd_f32(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int T, int D, int pattern, int l, int c, void* stream) {
  return attn_bwd<float>("st_sparse_attn_bwd_f32", q, k, v, out, lse, dout, dq, dk, dv, B, H, T,
                         D, pattern, l, c, nullptr, stream);
}

int st_sparse_attn_fwd_ex(int dtype, const void* q, const void* k, const void* v, void* out, float* lse, int B,
                          int H, int T, int D, int pattern, int l, int c, const int32_t* summary,
                          void* stream) {
  const char* fn = "st_sparse_attn_fwd_ex";
  switch (dtype) {
    case ST_BF16: return attn_fwd<bf16>(fn, q, k, v, out, lse, B, H, T, D, pattern, l, c, summary, stream);
    case ST_F16: return attn_fwd<f16>(fn, q, k, v, out, lse, B, H, T, D, pattern, l, c, summary, stream);
    case ST_F32: return attn_fwd<float>(fn, q, k, v, out, lse, B, H, T, D, pattern, l, c, summary, stream);
    default: set_error(std::string(fn) + ": unknown dtype " + std::to_string(dtype)); return ST_ERR_INVALID;
  }
}

int st_sparse_attn_bwd_ex(int dtype, const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int H,
                          int T, int D, int pattern, int l, int c, const int32_t* summary, void* stream) {
  const char* fn = "st_sparse_attn_bwd_ex";
  switch (dtype) {
    case ST_BF16:
      return attn_bwd<bf16>(fn, q, k, v, out, lse, dout, dq, dk, dv, B, H, T, D, pattern, l, c, summary, stream);
    case ST_F16:
      return attn_bwd<f16>(fn, q, k, v, out, lse, dout, dq, dk, dv, B, H, T, D, pattern, l, c, summary, stream);
    case ST_F32:
      return attn_bwd<float>(fn, q, k, v, out, lse, dout, dq, dk, dv, B, H, T, D, pattern, l, c, summary,
                             stream);
    default: set_error(std::string(fn) + ": unknown dtype " + std::to_string(dtype)); return ST_ERR_INVALID;
  }
}

int st_sparse_attn_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* out,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int H,
                               int T, int D, int pattern, int l, int c, const int32_t* summary, void* stream) {
  const char* fn = "st_sparse_attn_bwd_noalloc";
  switch (dtype) {
    case ST_BF16:
      return attn_bwd<bf16>(fn, q, k, v, out, lse, dout, dq, dk, dv, B, H, T, D, pattern, l, c, summary, stream,
                            true);
    case ST_F16:
      return attn_bwd<f16>(fn, q, k, v, out, lse, dout, dq, dk, dv, B, H, T, D, pattern, l, c, summary, stream,
                           true);
    case ST_F32:
      return attn_bwd<float>(fn, q, k, v, out, lse, dout, dq, dk, dv, B, H, T, D, pattern, l, c, summary, stream,
                             true);
    default: set_error(std::string(fn) + ": unknown dtype " + std::to_string(dtype)); return ST_ERR_INVALID;
  }
}

int st_set_fwd_rows_per_wave(int rows) {
  if (rows != 0 && rows != 16 && rows != 32) {
    set_error("st_set_fwd_rows_per_wave: rows must be 0, 16 or 32, got " + std::to_string(rows));
    return ST_ERR_INVALID;
  }
  g_fwd_rows_per_wave.store(rows, std::memory_order_relaxed);
  return ST_OK;
}

int st_set_dkdv_keys_per_wave(int keys) {
  if (keys != 0 && keys != 16 && keys != 32) {
    set_error("st_set_dkdv_keys_per_wave: keys must be 0, 16 or 32, got " + std::to_string(keys));
    return ST_ERR_INVALID;
  }
  g_dkdv_keys_per_wave.store(keys, std::memory_order_relaxed);
  return ST_OK;
}

int st_timing_enable(int on) {
  std::lock_guard<std::mutex> lock(g_timing_mutex);
  g_timing_on = on != 0;
  return ST_OK;
}

int st_timing_read(const char* kernel, int64_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) {
    set_error("st_timing_read: null argument");
    return ST_ERR_INVALID;
  }
  int kid = -1;
  for (int i = 0; i < KID_COUNT; ++i)
    if (std::string(kernel) == kKernelNames[i]) kid = i;
  if (kid < 0) {
    set_error(std::string("st_timing_read: unknown kernel ") + kernel);
    return ST_ERR_INVALID;
  }
  std::lock_guard<std::mutex> lock(g_timing_mutex);
  const int rc = drain_records();
  if (rc != ST_OK) return rc;
  *launches = g_launches[kid];
  *total_ms = g_total_ms[kid];
  return ST_OK;
}

void st_timing_reset(void) {
  std::lock_guard<std::mutex> lock(g_timing_mutex);
  (void)drain_records();
  for (int i = 0; i < KID_COUNT; ++i) {
    g_launches[i] = 0;
    g_total_ms[i] = 0.0;
  }
}

void st_release(void) {
  std::lock_guard<std::mutex> lock(g_mutex);
  int current = 0;
  const bool have_device = hipGetDevice(&current) == hipSuccess;
  // kernels still queued may read a plan or the workspace: every device the
  // library holds memory on finishes its work before anything is freed
  if (have_device) {
    std::set<int> devices;
    for (const auto& kv : g_plans) devices.insert(kv.first.device);
    for (const auto& kv : g_workspace) devices.insert(kv.first);
    for (int d : devices)
      if (hipSetDevice(d) == hipSuccess) (void)hipDeviceSynchronize();
  }
  for (auto& kv : g_plans) {
    if (have_device) (void)hipSetDevice(kv.first.device);
    kv.second.reset();
  }
  g_plans.clear();
  g_plan_use.clear();
  for (auto& kv : g_workspace) {
    if (have_device) (void)hipSetDevice(kv.first);
    if (kv.second.p) (void)hipFree(kv.second.p);
    if (kv.second.done) (void)hipEventDestroy(kv.second.done);
  }
  g_workspace.clear();
  if (have_device) (void)hipSetDevice(current);
}

}  // extern "C"
