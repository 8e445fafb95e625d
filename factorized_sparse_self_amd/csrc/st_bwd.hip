// Recompute backward of sparse attention for gfx950.
//
// The attention weights are not kept from the forward; they are rebuilt from
// q, k and the row log-sum-exp when the gradients need them (nlp-lineage,
// "The idea", recomputation).  For L = <dO, O>:
//   p_tj = exp(s_tj - lse_t),  Delta_t = dO_t . O_t,
//   dp_tj = dO_t . v_j,        ds_tj = p_tj (dp_tj - Delta_t),
//   dq_t = sum_j ds_tj k_j / sqrt(D),  dk_j = sum_t ds_tj q_t / sqrt(D),
//   dv_j = sum_t p_tj dO_t.
// In the 16-bit kernels (bf16 or fp16 inputs) P and dS enter the dV, dK and
// dQ products in the input's type (fp32 accumulation); bf16 dV and dK add the
// low parts of P and dS for rows whose weights are large.  Delta for dk / dv
// is exact: the dq pass adds to dO . O (O rounded to the output type) the sum
// of its fp32 dS over the row's keys, which is the rounding's contribution.
// Kernels (one stream, in order):
//   pre   Delta for every row; zero dk / dv at positions no query attends
//         (fp32 only: the 16-bit dq kernel does both for its own rows)
//   dq    per row block over the CSR (no cross-item reduction)
//   dkdv  per key block over the CSC; key blocks with many row blocks are
//         split, each split writing fp32 partials
//   red   sums the partials of split key blocks
#include <type_traits>

#include "st_device.hpp"
#include "st_kernels.hpp"
#include "st_stage.hpp"

namespace st {

namespace {

// LDS ring stages of the 16-bit dk/dv pass (row blocks in flight = stages - 1)
#ifndef ST_DKDV_STAGES
#define ST_DKDV_STAGES 2
#endif
constexpr int kDkdvStages = ST_DKDV_STAGES;
// LDS ring stages of the 16-bit dq pass
#ifndef ST_DQ_STAGES
#define ST_DQ_STAGES 2
#endif
constexpr int kDqStages = ST_DQ_STAGES;

// fp32 path: tiles staged row-major in LDS (pitch D + 2 floats).
template <int D>
struct BwdLdsF32 {
  static constexpr int RP = D + 2;
  static constexpr int R_ELEMS = kBlock * RP;
};

template <int D>
__device__ __forceinline__ void stage_row_f32(const float* __restrict__ src, int p, int r, int ch,
                                              float* rows) {
  using L = BwdLdsF32<D>;
  float4 x = {0.f, 0.f, 0.f, 0.f};
  if (p >= 0) x = *(const float4*)(src + (size_t)p * D + ch * 4);
  float* d = rows + r * L::RP + ch * 4;
  *(float2*)d = make_float2(x.x, x.y);
  *(float2*)(d + 2) = make_float2(x.z, x.w);
}

// ---------------------------------------------------------------------------
// pre: Delta_t = sum_d dO_t,d O_t,d; zero dk / dv where no query attends.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_f32_kernel(BwdArgs a) {
  using TE = float;
  constexpr int VEC = 4;                // elements per 16-byte chunk
  constexpr int TPR = D / VEC;          // threads per row (power of two)
  const int64_t row = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / TPR;
  const int ch = threadIdx.x % TPR;
  const int64_t n_rows = (int64_t)a.BH * a.T;
  const bool valid = row < n_rows;
  float part = 0.f;
  if (valid) {
    const TE* o = (const TE*)a.o + row * D + ch * VEC;
    const TE* g = (const TE*)a.dout + row * D + ch * VEC;
#pragma unroll
    for (int i = 0; i < VEC; ++i) part += (float)o[i] * (float)g[i];
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) part += xor_shfl(part, m);
  if (!valid) return;
  if (ch == 0) a.ndelta[row] = -part;
  // (a merged head's own-window or own-block kind attends every key)
  if (a.out_mode != OUT_FINAL) return;
  const int bh = (int)(row / a.T), t = (int)(row - (int64_t)bh * a.T);
  const Geometry& g = a.kinds[(bh % a.H) & 1].geo;
  if (!position_is_key(g, t)) {
    store_zero16_nt((TE*)a.dk + row * D + ch * VEC);
    store_zero16_nt((TE*)a.dv + row * D + ch * VEC);
  }
}

// ---------------------------------------------------------------------------
// Stores of one gradient row (dq of a query, dk or dv of a key): ND runs of 4
// floats at element offsets 16 d (the lane's quarter of the row; `dst` and
// `carry` point at its first element), scaled by `scale`, written as the
// launch's OutMode says.
// ---------------------------------------------------------------------------
template <int ND, typename E>
__device__ __forceinline__ void store_grad_row(int mode, float* carry, E* dst, const f32x4* x, float scale) {
  if (mode == OUT_CARRY) {
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const f32x4 y = x[d] * scale;
      *(float4*)(carry + 16 * d) = make_float4(y[0], y[1], y[2], y[3]);
    }
    return;
  }
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    f32x4 y = x[d] * scale;
    if (mode == OUT_MERGE) {
      const float4 c = *(const float4*)(carry + 16 * d);
      y += (f32x4){c.x, c.y, c.z, c.w};
    }
    if constexpr (std::is_same<E, float>::value)
      *(float4*)(dst + 16 * d) = make_float4(y[0], y[1], y[2], y[3]);
    else
      *(typename Vec<E>::x4*)(dst + 16 * d) = to_x4<E>(y);
  }
}

// Store mode of the dk / dv row of key position p: in the first pass of a
// merged head, only keys that the second pass holds are carried; the others
// are final.
__device__ __forceinline__ int key_out_mode(const BwdArgs& a, int p) {
  if (a.out_mode != OUT_CARRY) return a.out_mode;
  const Geometry g1 = load_uniform(&a.kinds[1].geo);
  return position_is_key(g1, p) ? OUT_CARRY : OUT_FINAL;
}

// ---------------------------------------------------------------------------
// dq: per row block; 4 waves x 16 rows; loop over the CSR key blocks.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_f32_kernel(BwdArgs a) {
  using L = BwdLdsF32<D>;
  using TE = float;
  constexpr int NQ = D / 4;
  constexpr int ND = D / 16;
  __shared__ __attribute__((aligned(16))) float Ks[L::R_ELEMS];
  __shared__ __attribute__((aligned(16))) float Vs[L::R_ELEMS];

  const RowItem item = load_uniform(&a.dq_items[blockIdx.x]);
  if (item.qb < 0) return;  // schedule padding
  const int qb = item.qb, bh = item.bh;
  const KindDev kd = load_uniform(&a.kinds[item.kind]);
  const Geometry& g = kd.geo;
  const size_t base = (size_t)bh * a.T * D;
  const TE* __restrict__ Qg = (const TE*)a.q + base;
  const TE* __restrict__ Kg = (const TE*)a.k + base;
  const TE* __restrict__ Vg = (const TE*)a.v + base;
  const TE* __restrict__ Gg = (const TE*)a.dout + base;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int R = qb * kBlock + wave * 16 + li;
  const int t = row_position(g, R);
  int lo = 1, hi = 0;
  if (t >= 0) row_interval(g, R, t, lo, hi);
  const int wlo = wave_min(lo <= hi ? lo : 0x7fffffff);
  const int whi = wave_max(lo <= hi ? hi : -1);
  const bool wave_active = whi >= 0;
  float lse2 = 0.f, ndelta = 0.f;
  if (t >= 0 && lo <= hi) {
    lse2 = a.lse[(size_t)bh * a.T + t] * kLog2e;
    ndelta = a.ndelta[(size_t)bh * a.T + t];
  }

  float qop[NQ], gop[NQ];
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    qop[s] = (t >= 0) ? Qg[(size_t)t * D + 4 * s + lg] : 0.f;
    gop[s] = (t >= 0) ? Gg[(size_t)t * D + 4 * s + lg] : 0.f;
  }
  f32x4 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.sl2;

  const int e0 = as_const(kd.row_ptr)[qb], e1 = as_const(kd.row_ptr)[qb + 1];
  for (int e = e0; e < e1; ++e) {
    const int kb = kd.col_idx[e];
    const bool full = kd.flags[e] != 0;
    __syncthreads();
    constexpr int CH = D / 4;
    for (int u = tid; u < kBlock * CH; u += kThreads) {
      const int r = u / CH, ch = u - r * CH;
      const int p = key_position(g, kb * kBlock + r);
      stage_row_f32<D>(Kg, p, r, ch, Ks);
      stage_row_f32<D>(Vg, p, r, ch, Vs);
    }
    __syncthreads();
    if (!wave_active) continue;

    const int k0 = kb * kBlock;
    bool need[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      need[b] = full || (k0 + 16 * b <= whi && k0 + 16 * b + 15 >= wlo);

    f32x4 s[4], dp[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      s[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      dp[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (!need[b]) continue;
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        s[b] = mfma_f32(Ks[(16 * b + li) * L::RP + 4 * k + lg], qop[k], s[b]);
        dp[b] = mfma_f32(Vs[(16 * b + li) * L::RP + 4 * k + lg], gop[k], dp[b]);
      }
    }
    // ds = p * (dp - Delta), p rebuilt from lse; zero outside the row's run
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int Kk = k0 + 16 * b + 4 * lg + i;
        const bool in = full || (Kk >= lo && Kk <= hi);
        const float p = in ? fast_exp2(fmaf(s[b][i], sl2, -lse2)) : 0.f;
        s[b][i] = p * (dp[b][i] + ndelta);
      }
    // dq^T += K^T ds^T
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (!need[b]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < ND; ++d)
          acc[d] = mfma_f32(Ks[(16 * b + 4 * lg + i) * L::RP + 16 * d + li], s[b][i], acc[d]);
    }
  }
  if (t < 0) return;
  store_grad_row<ND>(a.out_mode, a.carry_dq + ((size_t)bh * a.T + t) * D + 4 * lg,
                     (TE*)a.dq + base + (size_t)t * D + 4 * lg, acc, a.scale);
}

// ---------------------------------------------------------------------------
// dkdv: per key block (or a split of its row blocks); 4 waves x 16 keys.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_f32_kernel(BwdArgs a) {
  using L = BwdLdsF32<D>;
  using TE = float;
  constexpr int NQ = D / 4;
  constexpr int ND = D / 16;
  __shared__ __attribute__((aligned(16))) float Qs[L::R_ELEMS];
  __shared__ __attribute__((aligned(16))) float Gs[L::R_ELEMS];
  __shared__ __attribute__((aligned(16))) float lse2s[kBlock];
  __shared__ __attribute__((aligned(16))) float dels[kBlock];
  __shared__ __attribute__((aligned(16))) int los[kBlock];
  __shared__ __attribute__((aligned(16))) int his[kBlock];

  const DkdvItem item = load_uniform(&a.dkdv_items[blockIdx.x]);
  if (item.kb < 0) return;  // schedule padding
  const int kb = item.kb, bh = item.bh;
  const KindDev kd = load_uniform(&a.kinds[item.kind]);
  const Geometry& g = kd.geo;
  const size_t base = (size_t)bh * a.T * D;
  const TE* __restrict__ Qg = (const TE*)a.q + base;
  const TE* __restrict__ Kg = (const TE*)a.k + base;
  const TE* __restrict__ Vg = (const TE*)a.v + base;
  const TE* __restrict__ Gg = (const TE*)a.dout + base;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int Kw0 = kb * kBlock + wave * 16;  // first key of this wave
  const int Kl = Kw0 + li;                  // this lane's key
  const int kp = key_position(g, Kl);

  float kop[NQ], vop[NQ];
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    kop[s] = (kp >= 0) ? Kg[(size_t)kp * D + 4 * s + lg] : 0.f;
    vop[s] = (kp >= 0) ? Vg[(size_t)kp * D + 4 * s + lg] : 0.f;
  }
  f32x4 dk[ND], dv[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    dk[d] = (f32x4){0.f, 0.f, 0.f, 0.f};
    dv[d] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = a.sl2;

  for (int e = item.e0; e < item.e1; ++e) {
    const int qb = kd.row_idx[e];
    const bool full = kd.csc_flags[e] != 0;
    __syncthreads();
    constexpr int CH = D / 4;
    for (int u = tid; u < kBlock * CH; u += kThreads) {
      const int r = u / CH, ch = u - r * CH;
      const int p = row_position(g, qb * kBlock + r);
      stage_row_f32<D>(Qg, p, r, ch, Qs);
      stage_row_f32<D>(Gg, p, r, ch, Gs);
    }
    if (tid < kBlock) {
      const int R = qb * kBlock + tid;
      const int t = row_position(g, R);
      int lo = 1, hi = 0;
      float l2 = 0.f, de = 0.f;
      if (t >= 0) {
        row_interval(g, R, t, lo, hi);
        if (lo <= hi) {
          l2 = a.lse[(size_t)bh * a.T + t] * kLog2e;
          de = a.ndelta[(size_t)bh * a.T + t];
        }
      }
      los[tid] = lo;
      his[tid] = hi;
      lse2s[tid] = l2;
      dels[tid] = de;
    }
    __syncthreads();

    // which 16-row blocks have a row whose run meets this wave's 16 keys
    const int rlo = los[lane], rhi = his[lane];
    const uint64_t hit = __ballot(rlo <= rhi && rlo <= Kw0 + 15 && rhi >= Kw0);
    bool need[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) need[b] = full || ((hit >> (16 * b)) & 0xffffull) != 0;
    if (!full && hit == 0) continue;

    // S = Q K^T and dP = dO V^T: lane holds rows 16b + 4lg + i of key Kl
    f32x4 s[4], dp[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      s[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      dp[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (!need[b]) continue;
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        s[b] = mfma_f32(Qs[(16 * b + li) * L::RP + 4 * k + lg], kop[k], s[b]);
        dp[b] = mfma_f32(Gs[(16 * b + li) * L::RP + 4 * k + lg], vop[k], dp[b]);
      }
    }
    // p and ds for each (row 16b + 4lg + i, key Kl)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r0 = 16 * b + 4 * lg;
      const float4 l2 = *(const float4*)(lse2s + r0);
      const float4 de = *(const float4*)(dels + r0);
      const int4 lo4 = *(const int4*)(los + r0);
      const int4 hi4 = *(const int4*)(his + r0);
      const float l2a[4] = {l2.x, l2.y, l2.z, l2.w};
      const float dea[4] = {de.x, de.y, de.z, de.w};
      const int loa[4] = {lo4.x, lo4.y, lo4.z, lo4.w};
      const int hia[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = full || (Kl >= loa[i] && Kl <= hia[i]);
        const float p = in ? fast_exp2(fmaf(s[b][i], sl2, -l2a[i])) : 0.f;
        s[b][i] = p;
        dp[b][i] = p * (dp[b][i] + dea[i]);
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (!need[b]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const int off = (16 * b + 4 * lg + i) * L::RP + 16 * d + li;
          dv[d] = mfma_f32(Gs[off], s[b][i], dv[d]);
          dk[d] = mfma_f32(Qs[off], dp[b][i], dk[d]);
        }
    }
  }

  if (item.slot < 0) {
    if (kp < 0) return;
    const int mode = key_out_mode(a, kp);
    const size_t off = ((size_t)bh * a.T + kp) * D + 4 * lg;
    store_grad_row<ND>(mode, a.carry_dk + off, (TE*)a.dk + off, dk, a.scale);
    store_grad_row<ND>(mode, a.carry_dv + off, (TE*)a.dv + off, dv, 1.f);
  } else {
    float* pk = a.partial + ((size_t)item.slot * 2) * kBlock * D + (wave * 16 + li) * D;
    float* pv = pk + kBlock * D;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const f32x4 x = dk[d] * a.scale;
      *(float4*)(pk + 16 * d + 4 * lg) = make_float4(x[0], x[1], x[2], x[3]);
      *(float4*)(pv + 16 * d + 4 * lg) = make_float4(dv[d][0], dv[d][1], dv[d][2], dv[d][3]);
    }
  }
}


// ---------------------------------------------------------------------------
// 16-bit dq and dk/dv.  As in the forward: the streamed blocks (K and V for dq;
// Q and dO with their lse, Delta and key runs for dk/dv) go straight from
// global memory into a ring of swizzled LDS stages (st_stage.hpp) with the
// next blocks' loads in flight (padding rows read as zeros); FULL blocks run
// without masks; every transposed MFMA operand (K^T, Q^T, dO^T) comes from
// LDS transpose reads.
// ---------------------------------------------------------------------------
// dq: a work item is a pair of 64-row blocks (LUT blocks 2pb and 2pb+1) and
// the union of their key-block lists; eight waves, 16 rows each (waves 0-3 the
// first block, 4-7 the second).  Every K and V block is staged once for both
// row blocks; a wave skips (uniformly) the blocks its own row block does not
// visit.
//
// Delta.  The dP accumulators start at -Delta_O, with Delta_O = dO . O from
// the stored (rounded) output.  The fp32 dS summed over a row's keys is then
// sum_j p_j dp_j - Delta_O, the rounding's share of Delta (the weights sum to
// 1), so Delta_O plus that sum is the exact Delta, which the dk/dv pass gets.
// A row with few keys (pairs with kPairLo) gives each of them a large weight,
// so its own dq needs the exact Delta and dS as hi + lo too: a row whose keys
// lie in one 64-key block forms the exact Delta from that block's sum before
// its dQ product (ROW_INBLOCK); for the other such rows (ROW_PRE) a pre-pass
// of this kernel (DQ_DELTA: no dQ product, no stores but Delta) computes it.
enum DqMode : int { DQ_MAIN = 0, DQ_DELTA = 1 };

// Threads of a 16-bit dq workgroup: eight waves over both row blocks of a pair,
// or at D = 128 (181 VGPRs: one eight-wave workgroup per CU) four waves over one
// row block of the pair, two workgroups per pair.
template <int D>
constexpr int dq_threads() { return D >= 128 ? 256 : kDqThreads; }

template <typename E, int D, int NS, int KC, int MODE>
__device__ __forceinline__ void bwd_dq_b16_body(const BwdArgs& a, const PairItem& item,
                                                unsigned char (*ring)[2][TileShape<D>::BYTES]) {
  using S = TileShape<D>;
  typedef typename Vec<E>::x8 V8;
  constexpr int NQ = D / 32, ND = D / 16, CH = D / 8;
  constexpr int NW = dq_threads<D>() / 64;  // waves
  // staging: SW waves each stage SR rows of every tile (SNI instructions)
  constexpr int SR = S::RPI <= kBlock / NW ? kBlock / NW : S::RPI;
  constexpr int SW = kBlock / SR, SNI = SR / S::RPI;
  constexpr int PER_TILE = 2 * SNI;  // loads per staging wave per block (K and V)
  const int bh = item.bh;
  const KindDev kd = load_uniform(&a.kinds[item.kind]);
  const GeoC<KC> g{kd.geo};
  const size_t base = (size_t)bh * a.T * D;
  const uint32_t head_bytes = (uint32_t)a.T * D * 2;
  const Rsrc rq = make_rsrc((const E*)a.q + base, head_bytes);
  const Rsrc rk = make_rsrc((const E*)a.k + base, head_bytes);
  const Rsrc rv = make_rsrc((const E*)a.v + base, head_bytes);
  const Rsrc rg = make_rsrc((const E*)a.dout + base, head_bytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  // row block 2pb + half, rows 16 sub + li
  const int half = NW == 8 ? (wave >> 2) : (int)((blockIdx.x >> 3) & 1), sub = wave & 3;
  const int qb = 2 * item.pb + half;
  const bool stager = wave % (NW / SW) == 0;
  const int swave = wave / (NW / SW);
  const StageRows<SNI, S::RPI> stage(g, true, SR * swave + lane / S::CH);
  const cptr<uint32_t> entries = as_const(kd.pair_entry);
  // LDS address of this wave's staging rows in stage 0's K tile (V follows at
  // +BYTES, stage s at +s*STAGE)
  constexpr uint32_t STAGE = 2 * S::BYTES;
  const uint32_t lds_rows = lds_address(&ring[0][0][SR * swave * S::RB]);
  auto issue = [&](uint32_t entry, int stg) {
    if (!stager) return;
    int p[SNI];
    stage.positions(g, true, (int)(entry & kPairBlockMask), p);
    stage_rows<D>(rk, lds_rows + stg * STAGE, SR * swave, lane, p);
    stage_rows<D>(rv, lds_rows + stg * STAGE + S::BYTES, SR * swave, lane, p);
  };
  // The first NS-1 key blocks are in flight while the rows' own operands load
  // (those loads are younger, so the compiler's waits for them cover the ring's
  // first blocks too, and no compiler wait lands inside the loop).
  const int e0 = item.e0, e1 = item.e1;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (e0 + j < e1) issue(j == 0 ? item.first : entries[e0 + j], j);

  const int t = block_position(g, false, qb, sub * 16 + li);
  int lo = 1, hi = 0;
  if (t >= 0) row_interval(g, qb * kBlock + sub * 16 + li, t, lo, hi);
  const bool row_live = lo <= hi;
  const int mlo = row_live ? lo : -(1 << 30);
  const uint32_t mspan = row_live ? (uint32_t)(hi - lo) : 0u;
  // Delta_O = dO_t . O_t: each of the row's four lanes holds a quarter of the
  // row of dO (the MFMA operand) and loads the same quarter of O (O is read
  // nowhere else in the backward: a non-temporal load)
  const Rsrc ro = make_rsrc((const E*)a.o + base, head_bytes);
  V8 qop[NQ], gop[NQ];
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    const uint32_t off = t >= 0 ? (uint32_t)(t * D + 32 * s + 8 * lg) * 2 : kOutOfRange;
    qop[s] = __builtin_bit_cast(V8, buf_load16(rq, off));
    gop[s] = __builtin_bit_cast(V8, buf_load16(rg, off));
    const V8 o8 = __builtin_bit_cast(V8, buf_load16_nt(ro, off));
#pragma unroll
    for (int i = 0; i < 8; ++i) dpart = fmaf((float)gop[s][i], (float)o8[i], dpart);
  }
  // (rows that attend nothing get 0: no pass reads them)
  float delta = row_live ? group4_sum(dpart) : 0.f;
  const float lse2 =
      row_live ? buf_load_f32(make_rsrc(a.lse + (size_t)bh * a.T, (uint32_t)a.T * 4), (uint32_t)t * 4) * kLog2e
               : 0.f;
  const bool lo_pair = MODE == DQ_MAIN && (item.flags & kPairLo) != 0;  // uniform
  float inblock = 0.f;  // 1: the row forms its exact Delta inside its one key block
  if (lo_pair && row_live) {
    const int rf = kd.row_flags[t];
    if (rf & ROW_PRE) delta = -a.ndelta_pre[(size_t)bh * a.T + t];
    if (rf & ROW_INBLOCK) inblock = 1.f;
  }
  // dP^T accumulates onto -Delta, so dS = P * acc (this lane's column is row t)
  const f32x4 ndelta4 = {-delta, -delta, -delta, -delta};
  // per-lane byte offsets of the MFMA operand reads inside a staged block:
  // row operand k at a_off ^ (64 k) (chunk 4k + lg), transposed read d at
  // t_off ^ (32 d) (chunk 2d + ...): the swizzle XORs only the chunk bits
  static_assert(4 * (NQ - 1) < CH && 2 * (ND - 1) < CH, "operand chunks inside a row");
  const int a_off = S::phys(li, lg);
  const int t_off = S::phys(4 * lg + (li >> 2), (li & 3) >> 1) + 8 * (li & 1);
  f32x4 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.sl2;
  // sum over the row's keys of dS against the Delta in use (fp32, before
  // rounding): the Delta for dk/dv is that Delta plus this sum
  float dsum = 0.f;

  // One code path for every block (PARTIAL blocks only add the mask), in two
  // copies: plain, and for pairs with rows of few keys.
  auto step = [&](auto lo_c, int e, int stg) __attribute__((always_inline)) {
    constexpr bool LO = decltype(lo_c)::value;
    const uint32_t entry = e == e0 ? item.first : entries[e];
    const int k0 = (int)(entry & kPairBlockMask) * kBlock;
    const uint32_t hbits = (entry >> (28 + 2 * half)) & 3u;  // this row block's visit / FULL bits
    wait_tiles_left<PER_TILE, NS - 2>(imin(NS - 2, e1 - 1 - e));
    __syncthreads();
    if (e + NS - 1 < e1) issue(entries[e + NS - 1], stg == 0 ? NS - 1 : stg - 1);
    if (!(hbits & kPairVisit)) return;  // the other row block's key block
    const unsigned char* Kt = ring[stg][0];
    const unsigned char* Vt = ring[stg][1];
    // S^T = K Q^T and dP^T - Delta = V dO^T - Delta
    f32x4 sc[4], dp[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      sc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      dp[b] = ndelta4;
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        sc[b] = mfma16(*(const V8*)(Kt + 16 * b * S::RB + (a_off ^ (64 * k))), qop[k], sc[b]);
        dp[b] = mfma16(*(const V8*)(Vt + 16 * b * S::RB + (a_off ^ (64 * k))), gop[k], dp[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[b][i] = fast_exp2(fmaf(sc[b][i], sl2, -lse2));
    if (!(hbits & kPairFull)) {
      const int m0 = k0 + 4 * lg - mlo;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((uint32_t)(m0 + 16 * b + i) > mspan) sc[b][i] = 0.f;
    }
    if constexpr (!LO) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[b][i] *= dp[b][i];
          dsum += sc[b][i];
        }
      if constexpr (MODE == DQ_MAIN) {
        // dQ^T += K^T dS^T
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const V8 ds8 = pack_b_operand<E>(sc[2 * kk], sc[2 * kk + 1]);
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const unsigned char* r = Kt + 32 * kk * S::RB + (t_off ^ (32 * d));
            const V8 ak = concat(lds_read_tr<E>((const E*)r), lds_read_tr<E>((const E*)(r + 16 * S::RB)));
            acc[d] = mfma16(ak, ds8, acc[d]);
          }
        }
      }
    } else {
      // dp <- dS against the Delta in use; sc keeps P
      float bs = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dp[b][i] *= sc[b][i];
          bs += dp[b][i];
        }
      // a ROW_INBLOCK row has all its keys in this block (else P = 0 here and
      // bs = 0): bs is then its exact Delta's difference from Delta_O
      const float corr = inblock * group4_sum(bs);
      dsum += bs;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) dp[b][i] = fmaf(-sc[b][i], corr, dp[b][i]);
      // dQ^T += K^T (dS_hi + dS_lo)^T
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const V8 ds8 = pack_b_operand<E>(dp[2 * kk], dp[2 * kk + 1]);
        f32x4 r0, r1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r0[i] = dp[2 * kk][i] - (float)ds8[i];
          r1[i] = dp[2 * kk + 1][i] - (float)ds8[4 + i];
        }
        const V8 ds8lo = pack_b_operand<E>(r0, r1);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const unsigned char* r = Kt + 32 * kk * S::RB + (t_off ^ (32 * d));
          const V8 ak = concat(lds_read_tr<E>((const E*)r), lds_read_tr<E>((const E*)(r + 16 * S::RB)));
          acc[d] = mfma16(ak, ds8, acc[d]);
          acc[d] = mfma16(ak, ds8lo, acc[d]);
        }
      }
    }
  };
  if (lo_pair) {
    for (int e = e0, stg = 0; e < e1; ++e, stg = (stg + 1 == NS) ? 0 : stg + 1) step(std::true_type(), e, stg);
  } else {
    for (int e = e0, stg = 0; e < e1; ++e, stg = (stg + 1 == NS) ? 0 : stg + 1) step(std::false_type(), e, stg);
  }
  wait_vmcnt<0>();  // no DMA may still be writing LDS when the workgroup ends
  const float dsum_row = group4_sum(dsum);
  if constexpr (MODE == DQ_DELTA) {
    // the pre-pass: exact -Delta of the item's rows (a merged head's second
    // pass adds its keys' share to the rows it holds; its first pass, whose
    // kind attends every position, wrote every row)
    if (t >= 0 && lg == 0) {
      if (a.out_mode != OUT_MERGE)
        a.ndelta_pre[(size_t)bh * a.T + t] = -(delta + dsum_row);
      else if (row_live)
        a.ndelta_pre[(size_t)bh * a.T + t] -= dsum_row;
    }
    return;
  } else {
    // -Delta (exact) and lse*log2(e) of every row for the dk/dv pass, which
    // runs after every dq pass: the first pass of a merged head writes them,
    // its second adds its own keys' sum to the rows it holds
    if (t >= 0 && lg == 0) {
      float* rv = a.rowvals + 2 * ((size_t)bh * a.T + t);
      if (a.out_mode != OUT_MERGE) {
        rv[0] = lse2;
        rv[1] = -(delta + dsum_row);
      } else if (row_live) {
        rv[1] -= dsum_row;
      }
    }
    // keys nobody attends (positions outside a summary head's key map) get
    // dk = dv = 0; each row block's positions cover every such position
    // (in a merged head the first pass writes them)
    if constexpr (KC == K_SUMMARY || KC == K_SUMMARY_R1) {
      if (a.out_mode == OUT_FINAL)
        for (int u = tid & 255; u < kBlock * CH; u += 256) {
          const int r = u / CH, ch = u % CH;
          const int tp = block_position(g, false, qb, r);
          // (an explicit summary set: one byte per position instead of a search of the set)
          if (tp >= 0 && (g.sigma ? (kd.row_flags[tp] & ROW_NOKEY) != 0 : !position_is_key(g, tp))) {
            store_zero16_nt((E*)a.dk + base + (size_t)tp * D + ch * 8);
            store_zero16_nt((E*)a.dv + base + (size_t)tp * D + ch * 8);
          }
        }
    }
    if (a.out_mode != OUT_CARRY) {
      // whole-line dq rows through LDS (free once every wave is past its last
      // block), non-temporal; a merged head's second pass adds the carried rows
      using Rows = RowStage<E, D, 16>;
      static_assert(NW * Rows::BYTES <= NS * 2 * S::BYTES, "row staging fits the ring");
      f32x4 y[ND];
#pragma unroll
      for (int d = 0; d < ND; ++d) y[d] = acc[d] * a.scale;
      if (a.out_mode == OUT_MERGE && t >= 0) {
        const float* c = a.carry_dq + ((size_t)bh * a.T + t) * D + 4 * lg;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const float4 cv = *(const float4*)(c + 16 * d);
          y[d] += (f32x4){cv.x, cv.y, cv.z, cv.w};
        }
      }
      __syncthreads();
      Rows rows(&ring[0][0][0] + wave * Rows::BYTES);
      rows.template put<ND>(0, li, lg, y, 1.f);
#pragma unroll
      for (int j = 0; j < Rows::ROUNDS; ++j) {
        const int tr = block_position(g, false, qb, sub * 16 + rows.row_of(lane, j));
        const u32x4 x = rows.get(lane, j);
        if (tr >= 0)
          __builtin_nontemporal_store(x, (u32x4*)((E*)a.dq + base + (size_t)tr * D + rows.col_of(lane, j)));
      }
      return;
    }
    if (t < 0) return;
    store_grad_row<ND>(a.out_mode, a.carry_dq + ((size_t)bh * a.T + t) * D + 4 * lg,
                       (E*)a.dq + base + (size_t)t * D + 4 * lg, acc, a.scale);
  }
}

// One kernel per pattern and mode; each workgroup branches once on its head's kind.
template <typename E, int D, int NS, int C0, int C1, int MODE>
__global__ __launch_bounds__(dq_threads<D>()) void bwd_dq_b16_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[NS][2][TileShape<D>::BYTES];
  // four-wave workgroups: the two of a pair are 8 ids apart, on the same XCD
  const unsigned idx = dq_threads<D>() == kDqThreads ? blockIdx.x : ((blockIdx.x >> 4) << 3) | (blockIdx.x & 7);
  const PairItem item = load_uniform(&a.dq_pairs[idx]);
  if (item.pb < 0) return;  // schedule padding
  if (C0 == C1 || item.kind == 0)
    bwd_dq_b16_body<E, D, NS, C0, MODE>(a, item, ring);
  else
    bwd_dq_b16_body<E, D, NS, C1, MODE>(a, item, ring);
}

// dk/dv: Q and dO blocks with their lse*log2(e) and Delta are staged by
// direct global->LDS loads into a ring of NS stages (st_stage.hpp), so the
// loads of NS-1 row blocks are in flight while one is computed; each row's
// key run (for masks) is computed and stored next to them.  A workgroup holds
// one 64-key block; each of its 4/KT waves holds 16*KT keys.  With KT = 2 a
// wave reads every Q and dO operand from LDS once for two 16-key tiles, which
// halves the LDS reads per key against KT = 1, at twice the accumulators and
// half the waves.  That pays where items are long and the CUs stay full
// (launches with many more items than the GPU holds); where short items and
// latency set the time, KT = 1's four waves do better.  The launcher picks.
template <int D, int KT>
struct DkdvStage {
  unsigned char q[TileShape<D>::BYTES];
  unsigned char g[TileShape<D>::BYTES];
  // 16-row sub-block b at [VS b, VS b + 32): lse*log2(e) of each row, then
  // -Delta; VS = 64 / KT (with KT = 1 the second half of each slot is unused)
  float vals[4 * 64 / KT];
  int lo[kBlock];       // masking base of each row
  int span[kBlock];     // masking span (unsigned)
};

template <typename E, int D, int NS, int KC, int KT>
__device__ __forceinline__ void bwd_dkdv_b16_body(const BwdArgs& a, const DkdvItem& item, DkdvStage<D, KT>* ring) {
  using S = TileShape<D>;
  typedef typename Vec<E>::x8 V8;
  constexpr int NQ = D / 32, ND = D / 16;
  constexpr int WR = 16 * KT;                   // rows staged, and keys held, per wave
  constexpr int VS = 64 / KT;                   // row-value slot stride of a 16-row sub-block
  constexpr int PER_TILE = 2 * KT * S::NI + 1;  // loads per wave per row block: Q, dO, and lse2 with Delta
  using Stage = DkdvStage<D, KT>;
  const int kb = item.kb, bh = item.bh;
  const KindDev kd = load_uniform(&a.kinds[item.kind]);
  const GeoC<KC> g{kd.geo};
  const size_t base = (size_t)bh * a.T * D;
  const uint32_t head_bytes = (uint32_t)a.T * D * 2;
  const Rsrc rq = make_rsrc((const E*)a.q + base, head_bytes);
  const Rsrc rk = make_rsrc((const E*)a.k + base, head_bytes);
  const Rsrc rv = make_rsrc((const E*)a.v + base, head_bytes);
  const Rsrc rg = make_rsrc((const E*)a.dout + base, head_bytes);
  const Rsrc rvals = make_rsrc(a.rowvals + 2 * (size_t)bh * a.T, (uint32_t)a.T * 8);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  int Kl[KT], kp[KT];  // kernel key and position of this lane's key in each 16-key tile
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    Kl[kt] = kb * kBlock + wave * WR + 16 * kt + li;
    kp[kt] = block_position(g, true, kb, wave * WR + 16 * kt + li);
  }
  V8 kop[KT][NQ], vop[KT][NQ];  // this wave's keys as MFMA B operands (from LDS, first block)
  int a_off[NQ], t_off[ND];
#pragma unroll
  for (int k = 0; k < NQ; ++k) a_off[k] = S::phys(li, 4 * k + lg);
#pragma unroll
  for (int d = 0; d < ND; ++d) t_off[d] = S::phys(4 * lg + (li >> 2), 2 * d + ((li & 3) >> 1)) + 8 * (li & 1);
  f32x4 dk[KT][ND], dv[KT][ND];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int d = 0; d < ND; ++d) dk[kt][d] = dv[kt][d] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.sl2;

  // The row whose values (and key run) this lane fetches: lanes 32 h + i and
  // 32 h + 16 + i both take row i of the wave's sub-block h (the first its
  // lse*log2(e), the second its -Delta); with KT = 1 lanes 32..63 repeat 0..31.
  const int vh = (lane >> 5) % KT;
  const bool vlane = (lane >> 5) < KT;
  const int vrow = WR * wave + 16 * vh + li;
  const StageRows<KT * S::NI, S::RPI> stage(g, false, WR * wave + lane / S::CH);
  const StageRows<1, kBlock> stage_own(g, false, vrow);
  const cptr<uint32_t> entries = as_const(kd.csc_entry);
  // LDS addresses, in stage 0, of this wave's Q rows (dO follows at +BYTES)
  // and of its row values; stage s at +s*sizeof(Stage)
  static_assert(offsetof(Stage, g) - offsetof(Stage, q) == S::BYTES, "stage layout");
  const uint32_t lds_rows = lds_address(&ring[0].q[WR * wave * S::RB]);
  const uint32_t lds_vals = lds_address(&ring[0].vals[VS * KT * wave]);
  auto issue = [&](int e, int stg) {
    const uint32_t ent = entries[e];
    const int qb = (int)(ent & ~kFullBit);
    const uint32_t so = stg * (uint32_t)sizeof(Stage);
    int p[KT * S::NI];
    stage.positions(g, false, qb, p);
    stage_rows<D>(rq, lds_rows + so, WR * wave, lane, p);
    stage_rows<D>(rg, lds_rows + so + S::BYTES, WR * wave, lane, p);
    int tp[1];
    stage_own.positions(g, false, qb, tp);
    // a FULL block's rows are all real and attend every key of the block: no
    // key runs to form or store (its step applies no mask)
    bool live = true;
    if (!(ent & kFullBit)) {
      int lo = 1, hi = 0;
      if (tp[0] >= 0) row_interval(g, qb * kBlock + vrow, tp[0], lo, hi);
      live = lo <= hi;
      if (vlane && !(lane & 16)) {
        ring[stg].lo[vrow] = live ? lo : -(1 << 30);
        ring[stg].span[vrow] = live ? hi - lo : 0;
      }
    }
    // one load for both values (adjacent in the workspace); lanes without a
    // row write zeros
    lds_dma<4>(rvals, lds_vals + so, (vlane && live) ? (uint32_t)tp[0] * 8 + ((lane & 16) ? 4u : 0u) : kOutOfRange);
  };

  // The key block's K and V rows go through the last ring stage (free until
  // the first iteration refills it), ahead of the first NS-1 row blocks, so
  // every global load of the kernel is a ring DMA.
  if (item.e0 < item.e1) {
    const StageRows<KT * S::NI, S::RPI> kstage(g, true, WR * wave + lane / S::CH);
    int p[KT * S::NI];
    kstage.positions(g, true, kb, p);
    stage_rows<D>(rk, lds_rows + (NS - 1) * (uint32_t)sizeof(Stage), WR * wave, lane, p);
    stage_rows<D>(rv, lds_rows + (NS - 1) * (uint32_t)sizeof(Stage) + S::BYTES, WR * wave, lane, p);
  }
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (item.e0 + j < item.e1) issue(item.e0 + j, j);
  // One code path for every block (PARTIAL blocks only add the mask), in two
  // copies: with and without the low part of P in dV.
  auto step = [&](auto with_lo, int e, int stg) __attribute__((always_inline)) {
    constexpr bool LO = decltype(with_lo)::value;
    const bool full = (entries[e] & kFullBit) != 0;
    wait_tiles_left<PER_TILE, NS - 2>(imin(NS - 2, item.e1 - 1 - e));
    __syncthreads();
    if (e == item.e0) {
      // this wave's K/V rows (its own DMA, complete with the first block)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
          kop[kt][k] = *(const V8*)(ring[NS - 1].q + (WR * wave + 16 * kt) * S::RB + a_off[k]);
          vop[kt][k] = *(const V8*)(ring[NS - 1].g + (WR * wave + 16 * kt) * S::RB + a_off[k]);
        }
      // the reads must land before the DMA below refills that stage
      wait_lgkmcnt0();
    }
    if (e + NS - 1 < item.e1) issue(e + NS - 1, stg == 0 ? NS - 1 : stg - 1);
    const Stage& st = ring[stg];
    // The block's 64 rows as NG groups of 16-row sub-blocks: one group with
    // P and dS in the input type; two with their low parts too, or with two
    // key tiles, so that the operands fit the registers.
    constexpr int NG = (LO || KT > 1) ? 2 : 1, NB = 4 / NG;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      // S = Q K^T, and dP - Delta = dO V^T - Delta with the accumulators
      // starting at -Delta of rows 16b + 4lg + i; each Q and dO operand read
      // serves every key tile
      f32x4 sc[KT][NB], dp[KT][NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int b = gi * NB + j;
        const f32x4 nd = *(const f32x4*)(&st.vals[VS * b + 16 + 4 * lg]);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          sc[kt][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
          dp[kt][j] = nd;
        }
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
          const V8 qa = *(const V8*)(st.q + 16 * b * S::RB + a_off[k]);
          const V8 ga = *(const V8*)(st.g + 16 * b * S::RB + a_off[k]);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            sc[kt][j] = mfma16(qa, kop[kt][k], sc[kt][j]);
            dp[kt][j] = mfma16(ga, vop[kt][k], dp[kt][j]);
          }
        }
      }
      // rows 16b + 4lg + i of this lane's values
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int b = gi * NB + j;
        const float4 l2 = *(const float4*)(&st.vals[VS * b + 4 * lg]);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          sc[kt][j][0] = fast_exp2(fmaf(sc[kt][j][0], sl2, -l2.x));
          sc[kt][j][1] = fast_exp2(fmaf(sc[kt][j][1], sl2, -l2.y));
          sc[kt][j][2] = fast_exp2(fmaf(sc[kt][j][2], sl2, -l2.z));
          sc[kt][j][3] = fast_exp2(fmaf(sc[kt][j][3], sl2, -l2.w));
        }
      }
      if (!full) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int b = gi * NB + j;
          const int4 lo4 = *(const int4*)(&st.lo[16 * b + 4 * lg]);
          const int4 sp4 = *(const int4*)(&st.span[16 * b + 4 * lg]);
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            if ((uint32_t)(Kl[kt] - lo4.x) > (uint32_t)sp4.x) sc[kt][j][0] = 0.f;
            if ((uint32_t)(Kl[kt] - lo4.y) > (uint32_t)sp4.y) sc[kt][j][1] = 0.f;
            if ((uint32_t)(Kl[kt] - lo4.z) > (uint32_t)sp4.z) sc[kt][j][2] = 0.f;
            if ((uint32_t)(Kl[kt] - lo4.w) > (uint32_t)sp4.w) sc[kt][j][3] = 0.f;
          }
        }
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int j = 0; j < NB; ++j) dp[kt][j] *= sc[kt][j];
#pragma unroll
      for (int jj = 0; jj < NB / 2; ++jj) {
        const int kk = gi * (NB / 2) + jj;  // 32-row step
        V8 p8[KT], ds8[KT], p8lo[KT], ds8lo[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          p8[kt] = pack_b_operand<E>(sc[kt][2 * jj], sc[kt][2 * jj + 1]);
          ds8[kt] = pack_b_operand<E>(dp[kt][2 * jj], dp[kt][2 * jj + 1]);
          if constexpr (LO) {
            f32x4 r0, r1, u0, u1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              r0[i] = sc[kt][2 * jj][i] - (float)p8[kt][i];
              r1[i] = sc[kt][2 * jj + 1][i] - (float)p8[kt][4 + i];
              u0[i] = dp[kt][2 * jj][i] - (float)ds8[kt][i];
              u1[i] = dp[kt][2 * jj + 1][i] - (float)ds8[kt][4 + i];
            }
            p8lo[kt] = pack_b_operand<E>(r0, r1);
            ds8lo[kt] = pack_b_operand<E>(u0, u1);
          }
        }
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const unsigned char* rg0 = st.g + 32 * kk * S::RB + t_off[d];
          const unsigned char* rq0 = st.q + 32 * kk * S::RB + t_off[d];
          const V8 ag = concat(lds_read_tr<E>((const E*)rg0), lds_read_tr<E>((const E*)(rg0 + 16 * S::RB)));
          const V8 aq = concat(lds_read_tr<E>((const E*)rq0), lds_read_tr<E>((const E*)(rq0 + 16 * S::RB)));
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            dv[kt][d] = mfma16(ag, p8[kt], dv[kt][d]);
            if constexpr (LO) dv[kt][d] = mfma16(ag, p8lo[kt], dv[kt][d]);
            dk[kt][d] = mfma16(aq, ds8[kt], dk[kt][d]);
            if constexpr (LO) dk[kt][d] = mfma16(aq, ds8lo[kt], dk[kt][d]);
          }
        }
      }
    }
  };
  // bf16 carries P to dV and dS to dK as hi + lo for the row blocks whose rows
  // attend few keys (entries [e0, e_lo): along a key block's CSC list the rows'
  // key counts only grow).  Such rows give a key large weights, and the bf16
  // rounding of a large weight (relative 2^-9) summed over the many rows that
  // share the key can add up past the error bound; rows with many keys spread
  // their weights thinly.  fp16 rounds 8 times finer and needs no low part.
  constexpr bool kPLo = std::is_same<E, bf16>::value;
  if constexpr (kPLo) {
    int e = item.e0, stg = 0;
    for (; e < imin(item.e_lo, item.e1); ++e, stg = (stg + 1 == NS) ? 0 : stg + 1) step(std::true_type(), e, stg);
    for (; e < item.e1; ++e, stg = (stg + 1 == NS) ? 0 : stg + 1) step(std::false_type(), e, stg);
  } else {
    for (int e = item.e0, stg = 0; e < item.e1; ++e, stg = (stg + 1 == NS) ? 0 : stg + 1)
      step(std::false_type(), e, stg);
  }
  wait_vmcnt<0>();  // no DMA may still be writing LDS when the workgroup ends

  if (item.slot < 0 && a.out_mode != OUT_CARRY) {
    // whole-line dk and dv rows through LDS (free once every wave is past its
    // last block), non-temporal; a merged head's second pass adds the carried
    // rows (every key it holds was carried by the first pass)
    using Rows = RowStage<E, D, WR>;
    static_assert((4 / KT) * 2 * Rows::BYTES <= NS * sizeof(Stage), "row staging fits the ring");
    f32x4 yk[KT][ND], yv[KT][ND];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        yk[kt][d] = dk[kt][d] * a.scale;
        yv[kt][d] = dv[kt][d];
      }
    if (a.out_mode == OUT_MERGE) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        if (kp[kt] < 0) continue;
        const size_t off = ((size_t)bh * a.T + kp[kt]) * D + 4 * lg;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const float4 ck = *(const float4*)(a.carry_dk + off + 16 * d);
          const float4 cv = *(const float4*)(a.carry_dv + off + 16 * d);
          yk[kt][d] += (f32x4){ck.x, ck.y, ck.z, ck.w};
          yv[kt][d] += (f32x4){cv.x, cv.y, cv.z, cv.w};
        }
      }
    }
    __syncthreads();
    unsigned char* wbuf = (unsigned char*)(void*)ring + wave * 2 * Rows::BYTES;
    Rows rk(wbuf), rv(wbuf + Rows::BYTES);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      rk.template put<ND>(kt, li, lg, yk[kt], 1.f);
      rv.template put<ND>(kt, li, lg, yv[kt], 1.f);
    }
#pragma unroll
    for (int j = 0; j < Rows::ROUNDS; ++j) {
      const int kr = block_position(g, true, kb, wave * WR + rk.row_of(lane, j));
      const u32x4 xk = rk.get(lane, j), xv = rv.get(lane, j);
      if (kr >= 0) {
        const size_t off = base + (size_t)kr * D + rk.col_of(lane, j);
        __builtin_nontemporal_store(xk, (u32x4*)((E*)a.dk + off));
        __builtin_nontemporal_store(xv, (u32x4*)((E*)a.dv + off));
      }
    }
    return;
  }
  if (item.slot < 0) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      if (kp[kt] < 0) continue;
      const int mode = key_out_mode(a, kp[kt]);
      const size_t off = ((size_t)bh * a.T + kp[kt]) * D + 4 * lg;
      store_grad_row<ND>(mode, a.carry_dk + off, (E*)a.dk + off, dk[kt], a.scale);
      store_grad_row<ND>(mode, a.carry_dv + off, (E*)a.dv + off, dv[kt], 1.f);
    }
  } else {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      float* pk = a.partial + ((size_t)item.slot * 2) * kBlock * D + (wave * WR + 16 * kt + li) * D;
      float* pv = pk + kBlock * D;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const f32x4 x = dk[kt][d] * a.scale;
        *(float4*)(pk + 16 * d + 4 * lg) = make_float4(x[0], x[1], x[2], x[3]);
        *(float4*)(pv + 16 * d + 4 * lg) = make_float4(dv[kt][d][0], dv[kt][d][1], dv[kt][d][2], dv[kt][d][3]);
      }
    }
  }
}

// At least three waves per SIMD (at most 168 VGPRs) with one key tile per
// wave (about 120 VGPRs at D <= 64, so four fit), two with two tiles (about
// 200; the LDS ring allows four workgroups per CU either way).
template <typename E, int D, int NS, int C0, int C1, int KT>
__global__ __launch_bounds__(256 / KT) __attribute__((amdgpu_waves_per_eu(KT == 1 ? 3 : 2, 8))) void bwd_dkdv_b16_kernel(
    BwdArgs a) {
  __shared__ __attribute__((aligned(16))) DkdvStage<D, KT> ring[NS];
  const DkdvItem item = load_uniform(&a.dkdv_items[blockIdx.x]);
  if (item.kb < 0) return;  // schedule padding
  if (C0 == C1 || item.kind == 0)
    bwd_dkdv_b16_body<E, D, NS, C0, KT>(a, item, ring);
  else
    bwd_dkdv_b16_body<E, D, NS, C1, KT>(a, item, ring);
}

// ---------------------------------------------------------------------------
// red: sum the fp32 partials of a split key block and store dk / dv.
// ---------------------------------------------------------------------------
template <typename TE, int D>
__global__ __launch_bounds__(kThreads) void bwd_reduce_kernel(BwdArgs a) {
  // kParts workgroups per split key block, one float4 of dk or dv per thread
  constexpr int CH = D / 4;
  constexpr int kParts = 2 * kBlock * CH / kThreads;
  const ReduceItem item = load_uniform(&a.red_items[blockIdx.x / kParts]);
  if (item.kb < 0) return;  // schedule padding
  const KindDev kd = load_uniform(&a.kinds[item.kind]);
  const size_t base = (size_t)item.bh * a.T * D;
  const int u = (blockIdx.x % kParts) * kThreads + threadIdx.x;
  const int which = u / (kBlock * CH);  // 0 = dk, 1 = dv
  const int r = (u / CH) % kBlock, ch = u % CH;
  const int kp = block_position(kd.geo, true, item.kb, r);
  if (kp < 0) return;
  // the item's partials, eight loads in flight at a time (a buffer over its
  // slots: loads past the last slot return zeros, which add nothing), summed
  // in slot order
  constexpr int U = 8;
  constexpr uint32_t kSlotBytes = 2u * kBlock * D * 4;
  const Rsrc src = make_rsrc(a.partial + (size_t)item.slot0 * 2 * kBlock * D, (uint32_t)item.nsplit * kSlotBytes);
  const uint32_t off = (uint32_t)((which * kBlock + r) * D + ch * 4) * 4;
  float4 s = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < item.nsplit; j0 += U) {
    uint4 x[U];
#pragma unroll
    for (int i = 0; i < U; ++i) x[i] = buf_load16(src, (uint32_t)(j0 + i) * kSlotBytes + off);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      s.x += __uint_as_float(x[i].x);
      s.y += __uint_as_float(x[i].y);
      s.z += __uint_as_float(x[i].z);
      s.w += __uint_as_float(x[i].w);
    }
  }
  TE* dst = (TE*)(which ? a.dv : a.dk) + base + (size_t)kp * D + ch * 4;
  const f32x4 x[1] = {(f32x4){s.x, s.y, s.z, s.w}};
  store_grad_row<1>(key_out_mode(a, kp), (which ? a.carry_dv : a.carry_dk) + base + (size_t)kp * D + ch * 4, dst,
                    x, 1.f);
}

}  // namespace

template <typename TE, int D>
hipError_t launch_bwd_delta(const BwdArgs& a, int n_items, hipStream_t stream) {
  if constexpr (!Is16<TE>::value) {
    return hipErrorInvalidValue;  // the fp32 path takes Delta from its fp32 output
  } else {
    if (n_items <= 0) return hipSuccess;
    timing_begin(KID_DELTA, stream);
    const hipError_t err = with_kind_codes(a.pattern, [&](auto c0, auto c1, auto) {
      hipLaunchKernelGGL((bwd_dq_b16_kernel<TE, D, kDqStages, decltype(c0)::value, decltype(c1)::value, DQ_DELTA>),
                         dim3(n_items * (kDqThreads / dq_threads<D>())), dim3(dq_threads<D>()), 0, stream, a);
      return hipGetLastError();
    });
    timing_end(KID_DELTA, stream);
    return err;
  }
}

template <typename TE, int D>
hipError_t launch_bwd_dq(const BwdArgs& a, int n_dq, hipStream_t stream) {
  constexpr int TPR = D / (16 / sizeof(TE));
  const int64_t rows = (int64_t)a.BH * a.T;
  const int64_t pre_blocks = (rows * TPR + kThreads - 1) / kThreads;
  hipError_t err = hipSuccess;
  // 16-bit: the dq kernel computes Delta and the zero fill itself; it runs
  // before dk/dv, which reads Delta
  // (a merged head's second pass keeps the first pass's Delta)
  if (!Is16<TE>::value && a.out_mode != OUT_MERGE) {
    timing_begin(KID_PRE, stream);
    hipLaunchKernelGGL((bwd_pre_f32_kernel<D>), dim3((unsigned)pre_blocks), dim3(kThreads), 0, stream, a);
    err = hipGetLastError();
    timing_end(KID_PRE, stream);
    if (err != hipSuccess) return err;
  }
  if (n_dq > 0) {
    timing_begin(KID_DQ, stream);
    if constexpr (Is16<TE>::value) {
      err = with_kind_codes(a.pattern, [&](auto c0, auto c1, auto) {
        hipLaunchKernelGGL((bwd_dq_b16_kernel<TE, D, kDqStages, decltype(c0)::value, decltype(c1)::value, DQ_MAIN>),
                           dim3(n_dq * (kDqThreads / dq_threads<D>())), dim3(dq_threads<D>()), 0, stream, a);
        return hipGetLastError();
      });
    } else {
      hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), dim3(n_dq), dim3(kThreads), 0, stream, a);
      err = hipGetLastError();
    }
    timing_end(KID_DQ, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <typename TE, int D>
hipError_t launch_bwd_dkdv(const BwdArgs& a, int n_dkdv, int n_red, int keys_per_wave, hipStream_t stream) {
  hipError_t err = hipSuccess;
  if (n_dkdv > 0) {
    timing_begin(KID_DKDV, stream);
    if constexpr (Is16<TE>::value) {
      err = with_kind_codes(a.pattern, [&](auto c0, auto c1, auto) {
        constexpr int C0 = decltype(c0)::value, C1 = decltype(c1)::value;
        if constexpr (D <= 64) {
          if (keys_per_wave == 32) {
            hipLaunchKernelGGL((bwd_dkdv_b16_kernel<TE, D, kDkdvStages, C0, C1, 2>), dim3(n_dkdv), dim3(128), 0,
                               stream, a);
            return hipGetLastError();
          }
        }
        hipLaunchKernelGGL((bwd_dkdv_b16_kernel<TE, D, kDkdvStages, C0, C1, 1>), dim3(n_dkdv), dim3(kThreads), 0,
                           stream, a);
        return hipGetLastError();
      });
    } else {
      hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D>), dim3(n_dkdv), dim3(kThreads), 0, stream, a);
      err = hipGetLastError();
    }
    timing_end(KID_DKDV, stream);
    if (err != hipSuccess) return err;
  }
  if (n_red > 0) {
    timing_begin(KID_RED, stream);
    constexpr int kParts = 2 * kBlock * (D / 4) / kThreads;
    hipLaunchKernelGGL((bwd_reduce_kernel<TE, D>), dim3(n_red * kParts), dim3(kThreads), 0, stream, a);
    err = hipGetLastError();
    timing_end(KID_RED, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template hipError_t launch_bwd_delta<bf16, 32>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dq<bf16, 32>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dkdv<bf16, 32>(const BwdArgs&, int, int, int, hipStream_t);
template hipError_t launch_bwd_delta<bf16, 64>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dq<bf16, 64>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dkdv<bf16, 64>(const BwdArgs&, int, int, int, hipStream_t);
template hipError_t launch_bwd_delta<bf16, 128>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dq<bf16, 128>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dkdv<bf16, 128>(const BwdArgs&, int, int, int, hipStream_t);
template hipError_t launch_bwd_delta<f16, 32>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dq<f16, 32>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dkdv<f16, 32>(const BwdArgs&, int, int, int, hipStream_t);
template hipError_t launch_bwd_delta<f16, 64>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dq<f16, 64>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dkdv<f16, 64>(const BwdArgs&, int, int, int, hipStream_t);
template hipError_t launch_bwd_delta<f16, 128>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dq<f16, 128>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dkdv<f16, 128>(const BwdArgs&, int, int, int, hipStream_t);
template hipError_t launch_bwd_delta<float, 32>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dq<float, 32>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dkdv<float, 32>(const BwdArgs&, int, int, int, hipStream_t);
template hipError_t launch_bwd_delta<float, 64>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dq<float, 64>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dkdv<float, 64>(const BwdArgs&, int, int, int, hipStream_t);
template hipError_t launch_bwd_delta<float, 128>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dq<float, 128>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd_dkdv<float, 128>(const BwdArgs&, int, int, int, hipStream_t);

}  // namespace st
