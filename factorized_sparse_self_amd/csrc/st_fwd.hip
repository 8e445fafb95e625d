// Fused sparse attention forward for gfx950.
//
// Computes, per head, out_t = softmax_{j in S(t)}(q_t . k_j / sqrt(D)) v_j and
// lse_t (nlp-lineage, "The notation"; llm-arch-kb "Sparse Transformer", §2,
// masked logits carry no mass).  Only the block pairs the LUT lists are
// visited (llm-arch-kb §2 "Per-layer cost": a block-sparse product, not a
// masked dense one); inside PARTIAL blocks each logit outside the row's key
// run is set to -inf.
//
// S^T = K Q^T runs on MFMA so that each lane holds logits of its own query;
// the online softmax keeps the running max / sum in registers (cross-lane only
// over the 4 lanes of a query); O^T += V^T P^T runs on MFMA.  The 16-bit kernel
// (bf16 or fp16 inputs) is the product path; the fp32 kernel serves fp32 inputs.
#include <type_traits>

#include "st_device.hpp"
#include "st_kernels.hpp"
#include "st_stage.hpp"

namespace st {

namespace {

// LDS ring stages of the 16-bit forward (blocks in flight = stages - 1)
#ifndef ST_FWD_STAGES
#define ST_FWD_STAGES 2
#endif
constexpr int kFwdStages = ST_FWD_STAGES;

// ---------------------------------------------------------------------------
// fp32 forward: fp32 MFMA (16x16x4) on K and V staged row-major in LDS.
// ---------------------------------------------------------------------------
template <int D>
struct FwdLdsF32 {
  static constexpr int P = D + 2;  // row pitch (floats) of the K and V tiles
  static constexpr int ELEMS = kBlock * P;
};

// Stage key block kb of K and V into LDS (zeros for padding keys).
template <int D>
__device__ __forceinline__ void stage_kv_f32(const float* __restrict__ K, const float* __restrict__ V,
                                             const Geometry& g, int kb, float* Ks, float* Vs) {
  using L = FwdLdsF32<D>;
  constexpr int CH = D / 4;
  for (int u = threadIdx.x; u < kBlock * CH; u += kThreads) {
    const int r = u / CH, ch = u - r * CH;
    const int p = key_position(g, kb * kBlock + r);
    float4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
    if (p >= 0) {
      kk = *(const float4*)(K + (size_t)p * D + ch * 4);
      vv = *(const float4*)(V + (size_t)p * D + ch * 4);
    }
    float* kd = Ks + r * L::P + ch * 4;
    float* vd = Vs + r * L::P + ch * 4;
    *(float2*)kd = make_float2(kk.x, kk.y);
    *(float2*)(kd + 2) = make_float2(kk.z, kk.w);
    *(float2*)vd = make_float2(vv.x, vv.y);
    *(float2*)(vd + 2) = make_float2(vv.z, vv.w);
  }
}

// a*b - c with the product rounded before the subtraction (never fused)
__device__ __forceinline__ float mul_unfused(float a, float b, float c) {
#pragma clang fp contract(off)
  return a * b - c;
}

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a) {
  using L = FwdLdsF32<D>;
  constexpr int NQ = D / 4;   // MFMA k-steps over D
  constexpr int ND = D / 16;  // 16-wide output column blocks
  __shared__ __attribute__((aligned(16))) float Ks[L::ELEMS];
  __shared__ __attribute__((aligned(16))) float Vs[L::ELEMS];

  const RowItem item = load_uniform(&a.items[blockIdx.x]);
  if (item.qb < 0) return;  // schedule padding
  const int qb = item.qb, bh = item.bh;
  const KindDev kd = load_uniform(&a.kinds[item.kind]);
  const Geometry& g = kd.geo;
  const size_t base = (size_t)bh * a.T * D;
  const float* __restrict__ Q = (const float*)a.q + base;
  const float* __restrict__ Kg = (const float*)a.k + base;
  const float* __restrict__ Vg = (const float*)a.v + base;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int R = qb * kBlock + wave * 16 + li;
  const int t = row_position(g, R);
  int lo = 1, hi = 0;
  if (t >= 0) row_interval(g, R, t, lo, hi);
  const int wlo = wave_min(lo <= hi ? lo : 0x7fffffff);
  const int whi = wave_max(lo <= hi ? hi : -1);
  const bool wave_active = whi >= 0;

  // Q operand (B of S^T = K Q^T): lane holds Q[t][4s + lg] of k-step s
  float qop[NQ];
#pragma unroll
  for (int s = 0; s < NQ; ++s) qop[s] = (t >= 0) ? Q[(size_t)t * D + 4 * s + lg] : 0.f;

  f32x4 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.sl2;

  const int e0 = as_const(kd.row_ptr)[qb], e1 = as_const(kd.row_ptr)[qb + 1];
  for (int e = e0; e < e1; ++e) {
    const int kb = kd.col_idx[e];
    const bool full = kd.flags[e] != 0;
    __syncthreads();
    stage_kv_f32<D>(Kg, Vg, g, kb, Ks, Vs);
    __syncthreads();
    if (!wave_active) continue;

    const int k0 = kb * kBlock;
    bool need[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) need[b] = full || (k0 + 16 * b <= whi && k0 + 16 * b + 15 >= wlo);

    // S^T = K Q^T, one 16x16 block per 16 keys
    f32x4 s[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      s[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (!need[b]) continue;
#pragma unroll
      for (int k = 0; k < NQ; ++k) s[b] = mfma_f32(Ks[(16 * b + li) * L::P + 4 * k + lg], qop[k], s[b]);
    }
    // mask: keys outside this row's run (also padding rows / keys) -> -inf
    if (!full) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int Kk = k0 + 16 * b + 4 * lg + i;
          if (Kk < lo || Kk > hi) s[b][i] = -INFINITY;
        }
    }
    // online softmax (running max in raw logit units, exp2 with folded scale)
    float mt = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[b][i]);
    mt = group4_max(mt);
    const float m_new = fmaxf(m_run, mt);
    // exponents as rounded products (never fused), so that the row's maximum
    // logit gets exp2(0) = 1 exactly: a row with one key returns v bit for bit
    const float mb = (m_new == -INFINITY) ? 0.f : mul_unfused(m_new, sl2, 0.f);
    const float alpha = fast_exp2(mul_unfused(m_run, sl2, mb));
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(mul_unfused(s[b][i], sl2, mb));
        s[b][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (!need[b]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < ND; ++d) acc[d] = mfma_f32(Vs[(16 * b + 4 * lg + i) * L::P + 16 * d + li], s[b][i], acc[d]);
    }
  }

  // epilogue: normalise, write O and lse (natural log)
  const float lsum = group4_sum(l_run);
  if (t < 0) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const float lse2 = lsum > 0.f ? m_run * sl2 + fast_log2(lsum) : -INFINITY;  // log2 units
  const size_t row = (size_t)bh * a.T + t;
  float* O = (float*)a.o + row * D;
  if (a.out_mode == OUT_CARRY) {
    // first pass of a merged head: keep the normalised output and lse
    float* C = a.carry_o + row * D;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const f32x4 o = acc[d] * inv;
      *(float4*)(C + 16 * d + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (lg == 0) a.carry_lse[row] = lse2;
    return;
  }
  if (a.out_mode == OUT_MERGE) {
    // softmax over both key sets: the two passes' outputs weighted by
    // 2^(L_p - L), L = log2(2^L0 + 2^L1) (a pass with no keys has L_p = -inf)
    const float lse0 = a.carry_lse[row];
    const float mx = fmaxf(lse0, lse2);
    const float w0 = mx == -INFINITY ? 0.f : fast_exp2(lse0 - mx);
    const float w1 = mx == -INFINITY ? 0.f : fast_exp2(lse2 - mx);
    const float sw = w0 + w1;
    const float s0 = sw > 0.f ? w0 / sw : 0.f, s1 = sw > 0.f ? w1 * inv / sw : 0.f;
    const float* C = a.carry_o + row * D;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const float4 c = *(const float4*)(C + 16 * d + 4 * lg);
      const f32x4 o = (f32x4){c.x, c.y, c.z, c.w} * s0 + acc[d] * s1;
      *(float4*)(O + 16 * d + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (lg == 0) a.lse[row] = (sw > 0.f ? mx + fast_log2(sw) : -INFINITY) * kLn2;
    return;
  }
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const f32x4 o = acc[d] * inv;
    *(float4*)(O + 16 * d + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
  }
  if (lg == 0) a.lse[row] = lse2 * kLn2;
}

// ---------------------------------------------------------------------------
// 16-bit (bf16 or fp16) forward.
//  * Work item = a pair of 64-row LUT blocks (128 kernel rows) of one head; it
//    walks the union of the two blocks' key-block lists.  The first half of
//    the waves own the first block, the second half the second; a wave owns
//    GW MFMA groups of 16 rows (two in four-wave workgroups, which share every
//    K and V operand read from LDS; one in eight-wave ones), and skips the key
//    blocks its own row block does not visit.
//  * K and V blocks are staged by direct global->LDS loads into a ring of NS
//    LDS stages (st_stage.hpp): the loads of the next NS-1 blocks are in
//    flight while a block is computed, and no registers hold them.  Padding
//    rows read as zeros.  One barrier per block.
//  * Every block takes one code path; PARTIAL blocks add the mask, one
//    unsigned compare per logit.
//  * The V^T operand of the P.V product comes from LDS transpose reads.
//  * Online softmax: the row sum is fp32 (lse must be the log of the exact
//    sum: the backward rebuilds P from it).  The running max is only raised
//    when a logit exceeds it by more than 2^8 in exp2 units; blocks where no
//    lane of the wave needs that skip the cross-lane max and the rescale.
// ---------------------------------------------------------------------------
template <typename E, int D, int NS, int KC, bool M, int GW>
__device__ __forceinline__ void fwd_b16_body(const FwdArgs& a, const PairItem& item,
                                              unsigned char (*ring)[2][TileShape<D>::BYTES]) {
  using S = TileShape<D>;
  typedef typename Vec<E>::x8 V8;
  constexpr int NQ = D / 32;           // MFMA k-steps over D
  constexpr int ND = D / 16;           // 16-wide output column blocks
  constexpr int NW = 8 / GW;  // waves: NW/2 per row block, 16*GW rows each
  // staging: SW waves each stage SR rows of every tile (SNI instructions)
  constexpr int SR = S::RPI <= kBlock / NW ? kBlock / NW : S::RPI;
  constexpr int SW = kBlock / SR, SNI = SR / S::RPI;
  constexpr int PER_TILE = 2 * SNI;  // loads per staging wave per block (K and V)
  const int pb = item.pb, bh = item.bh;
  const KindDev kd = load_uniform(&a.kinds[item.kind]);
  const GeoC<KC> g{kd.geo};
  const size_t base = (size_t)bh * a.T * D;
  const uint32_t head_bytes = (uint32_t)a.T * D * 2;
  const Rsrc rq = make_rsrc((const E*)a.q + base, head_bytes);
  const Rsrc rk = make_rsrc((const E*)a.k + base, head_bytes);
  const Rsrc rv = make_rsrc((const E*)a.v + base, head_bytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  // The first NW/2 waves take row block 2pb, the others 2pb+1; a wave owns
  // 16*GW rows, GW MFMA groups of 16 that share every K and V operand.
  // (unsigned: a signed division here costs the four-wave form 10-16 VGPRs)
  const unsigned uw = (unsigned)wave;
  const int half = (int)(uw / (NW / 2));
  const int qb = 2 * pb + half;
  const int r0 = (int)(uw % (NW / 2)) * 16 * GW;
  const bool stager = uw % (NW / SW) == 0;
  const int swave = (int)(uw / (NW / SW));
  int t[GW], mlo[GW];
  uint32_t mspan[GW];
#pragma unroll
  for (int G = 0; G < GW; ++G) {
    const int r = r0 + 16 * G + li;
    t[G] = block_position(g, false, qb, r);
    int lo = 1, hi = 0;
    if (t[G] >= 0) row_interval(g, qb * kBlock + r, t[G], lo, hi);
    // logit of kernel key K is masked when (unsigned)(K - mlo) > mspan
    mlo[G] = lo <= hi ? lo : -(1 << 30);
    mspan[G] = lo <= hi ? (uint32_t)(hi - lo) : 0u;
  }

  // per-lane byte offsets of the MFMA operand reads inside a staged block
  int a_off[NQ], t_off[ND];
#pragma unroll
  for (int k = 0; k < NQ; ++k) a_off[k] = S::phys(li, 4 * k + lg);
#pragma unroll
  for (int d = 0; d < ND; ++d) t_off[d] = S::phys(4 * lg + (li >> 2), 2 * d + ((li & 3) >> 1)) + 8 * (li & 1);

  V8 qop[GW][NQ];  // the groups' query rows as MFMA B operands (from LDS, first block)
  f32x4 acc[GW][ND];
#pragma unroll
  for (int G = 0; G < GW; ++G)
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[G][d] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.sl2;
  const float headroom = 8.0f / sl2;  // raw-logit growth allowed before a rescale
  float m_run[GW], l_run[GW];
#pragma unroll
  for (int G = 0; G < GW; ++G) {
    m_run[G] = -INFINITY;
    l_run[G] = 0.f;
  }

  const StageRows<SNI, S::RPI> stage(g, true, SR * swave + lane / S::CH);
  const cptr<uint32_t> entries = as_const(kd.pair_entry);
  // LDS address of this wave's 16 staging rows in stage 0's K tile (V follows
  // at +BYTES, stage s at +s*STAGE)
  constexpr uint32_t STAGE = 2 * S::BYTES;
  const uint32_t lds_rows = lds_address(&ring[0][0][SR * swave * S::RB]);
  auto issue = [&](uint32_t entry, int stg) {
    if (!stager) return;
    int p[SNI];
    stage.positions(g, true, (int)(entry & kPairBlockMask), p);
    stage_rows<D>(rk, lds_rows + stg * STAGE, SR * swave, lane, p);
    stage_rows<D>(rv, lds_rows + stg * STAGE + S::BYTES, SR * swave, lane, p);
  };

  const int e0 = item.e0, e1 = item.e1;
  // The two row blocks' Q rows go through the last ring stage (free until the
  // first iteration refills it: row block 2pb in the K tile, 2pb+1 in the V
  // tile), ahead of the first NS-1 key blocks, so every global load of the
  // loop is a ring DMA.
  if (e0 < e1 && stager) {
    const StageRows<SNI, S::RPI> qstage(g, false, SR * swave + lane / S::CH);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      int p[SNI];
      qstage.positions(g, false, 2 * pb + hb, p);
      stage_rows<D>(rq, lds_rows + (NS - 1) * STAGE + hb * S::BYTES, SR * swave, lane, p);
    }
  }
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (e0 + j < e1) issue(j == 0 ? item.first : entries[e0 + j], j);
  for (int e = e0, stg = 0; e < e1; ++e, stg = (stg + 1 == NS) ? 0 : stg + 1) {
    const uint32_t entry = e == e0 ? item.first : entries[e];
    const int k0 = (int)(entry & kPairBlockMask) * kBlock;
    const uint32_t hbits = (entry >> (28 + 2 * half)) & 3u;  // this row block's visit / FULL bits
    wait_tiles_left<PER_TILE, NS - 2>(imin(NS - 2, e1 - 1 - e));
    __syncthreads();
    if (e == e0) {
      // the wave's own rows, staged by all four waves: complete after the barrier
      const unsigned char* qt = ring[NS - 1][half] + r0 * S::RB;
#pragma unroll
      for (int G = 0; G < GW; ++G)
#pragma unroll
        for (int k = 0; k < NQ; ++k) qop[G][k] = *(const V8*)(qt + 16 * G * S::RB + a_off[k]);
      // every wave's reads must land before any wave's DMA below refills
      // that stage (waves read rows that other waves staged)
      wait_lgkmcnt0();
      __syncthreads();
    }
    if (e + NS - 1 < e1) issue(entries[e + NS - 1], stg == 0 ? NS - 1 : stg - 1);
    if (!(hbits & kPairVisit)) continue;  // the other row block's key block
    const unsigned char* Kt = ring[stg][0];
    const unsigned char* Vt = ring[stg][1];

    // S^T = K Q^T for both groups: each K operand read serves two MFMAs
    f32x4 sc[GW][4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int G = 0; G < GW; ++G) sc[G][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        const V8 ka = *(const V8*)(Kt + 16 * b * S::RB + a_off[k]);
#pragma unroll
        for (int G = 0; G < GW; ++G) sc[G][b] = mfma16(ka, qop[G][k], sc[G][b]);
      }
    }
    if (!(hbits & kPairFull)) {
      // key k0 + 16b + 4lg + i is outside the row's run when
      // (unsigned)(key - mlo) > mspan
#pragma unroll
      for (int G = 0; G < GW; ++G) {
        const int m0 = k0 + 4 * lg - mlo[G];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((uint32_t)(m0 + 16 * b + i) > mspan[G]) sc[G][b][i] = -INFINITY;
      }
    }
    float lm[GW];
#pragma unroll
    for (int G = 0; G < GW; ++G) {
      lm[G] = fmaxf(fmaxf(sc[G][0][0], sc[G][0][1]), fmaxf(sc[G][0][2], sc[G][0][3]));
#pragma unroll
      for (int b = 1; b < 4; ++b)
        lm[G] = fmaxf(fmaxf(lm[G], fmaxf(sc[G][b][0], sc[G][b][1])), fmaxf(sc[G][b][2], sc[G][b][3]));
    }
    bool need = lm[0] > m_run[0] + headroom;
#pragma unroll
    for (int G = 1; G < GW; ++G) need = need || lm[G] > m_run[G] + headroom;
    if (wave_any(need)) {
#pragma unroll
      for (int G = 0; G < GW; ++G) {
        const float mt = group4_max(lm[G]);
        const bool raise = mt > m_run[G] + headroom;
        // raising rows scale by exp2((old - new) max), 0 when the old max is
        // -inf; the others keep their sums (factor exactly 1, never -inf - -inf)
        const float alpha = raise ? fast_exp2((m_run[G] - mt) * sl2) : 1.f;
#pragma unroll
        for (int d = 0; d < ND; ++d) acc[G][d] *= alpha;
        l_run[G] *= alpha;
        m_run[G] = raise ? mt : m_run[G];
      }
    }
    V8 pb8[GW][2];
#pragma unroll
    for (int G = 0; G < GW; ++G) {
      const float mb = (m_run[G] == -INFINITY) ? 0.f : m_run[G] * sl2;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[G][b][i] = fast_exp2(fmaf(sc[G][b][i], sl2, -mb));
          l_run[G] += sc[G][b][i];
        }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) pb8[G][kk] = pack_b_operand<E>(sc[G][2 * kk], sc[G][2 * kk + 1]);
    }
    // O^T += V^T P^T for both groups: each V^T operand read serves two MFMAs
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const unsigned char* r = Vt + 32 * kk * S::RB + t_off[d];
        const V8 av = concat(lds_read_tr<E>((const E*)r), lds_read_tr<E>((const E*)(r + 16 * S::RB)));
#pragma unroll
        for (int G = 0; G < GW; ++G) acc[G][d] = mfma16(av, pb8[G][kk], acc[G][d]);
      }
  }
  wait_vmcnt<0>();  // no DMA may still be writing LDS when the workgroup ends

  if (!M || a.out_mode != OUT_CARRY) {
    // whole-line output rows through LDS (free once every wave is past its
    // last block); ordinary stores, since the backward reads O again.  The
    // second pass of a merged head first combines its rows with the carried
    // ones: softmax over both key sets, weights exp2(L_p - L) of the two
    // passes' outputs, L = log2(2^L0 + 2^L1) (a pass with no keys has L_p = -inf)
    using Rows = RowStage<E, D, 16 * GW>;
    static_assert(NW * Rows::BYTES <= NS * 2 * S::BYTES, "row staging fits the ring");
    __syncthreads();
    Rows rows(&ring[0][0][0] + wave * Rows::BYTES);
#pragma unroll
    for (int G = 0; G < GW; ++G) {
      const float lsum = group4_sum(l_run[G]);
      // the output is rounded to 16 bits, so the hardware reciprocal (1 ulp) suffices
      const float inv = lsum > 0.f ? __builtin_amdgcn_rcpf(lsum) : 0.f;
      const float lse2 = lsum > 0.f ? fmaf(m_run[G], sl2, fast_log2(lsum)) : -INFINITY;  // log2 units
      bool merged = false;
      if constexpr (M) merged = a.out_mode == OUT_MERGE;
      if (merged) {
        f32x4 y[ND];
#pragma unroll
        for (int d = 0; d < ND; ++d) y[d] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (t[G] >= 0) {
          const size_t row = (size_t)bh * a.T + t[G];
          const float lse0 = a.carry_lse[row];
          const float mx = fmaxf(lse0, lse2);
          const float w0 = mx == -INFINITY ? 0.f : fast_exp2(lse0 - mx);
          const float w1 = mx == -INFINITY ? 0.f : fast_exp2(lse2 - mx);
          const float sw = w0 + w1;
          const float isw = sw > 0.f ? __builtin_amdgcn_rcpf(sw) : 0.f;
          const float s0 = w0 * isw, s1 = w1 * inv * isw;
          const float* C = a.carry_o + row * D;
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const float4 c = *(const float4*)(C + 16 * d + 4 * lg);
            const f32x4 c4 = {c.x, c.y, c.z, c.w};
            // explicit fma: the same operations in every instantiation of
            // the kernel (the compiler may contract a * b + c * d either way)
            const f32x4 c0 = c4 * s0;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[d][i] = fmaf(acc[G][d][i], s1, c0[i]);
          }
          if (lg == 0) a.lse[row] = (sw > 0.f ? mx + fast_log2(sw) : -INFINITY) * kLn2;
        }
        rows.template put<ND>(G, li, lg, y, 1.f);
      } else {
        rows.template put<ND>(G, li, lg, acc[G], inv);
        if (t[G] >= 0 && lg == 0) a.lse[(size_t)bh * a.T + t[G]] = lse2 * kLn2;
      }
    }
#pragma unroll
    for (int j = 0; j < Rows::ROUNDS; ++j) {
      const int tr = block_position(g, false, qb, r0 + rows.row_of(lane, j));
      const u32x4 x = rows.get(lane, j);
      if (tr >= 0) *(u32x4*)((E*)a.o + base + (size_t)tr * D + rows.col_of(lane, j)) = x;
    }
    return;
  }

  // first pass of a merged head: keep the normalised fp32 output and lse
#pragma unroll
  for (int G = 0; G < GW; ++G) {
    const float lsum = group4_sum(l_run[G]);
    if (t[G] < 0) continue;
    const float inv = lsum > 0.f ? __builtin_amdgcn_rcpf(lsum) : 0.f;
    const float lse2 = lsum > 0.f ? fmaf(m_run[G], sl2, fast_log2(lsum)) : -INFINITY;  // log2 units
    const size_t row = (size_t)bh * a.T + t[G];
    float* C = a.carry_o + row * D;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const f32x4 o = acc[G][d] * inv;
      *(float4*)(C + 16 * d + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (lg == 0) a.carry_lse[row] = lse2;
  }
}

}  // namespace

// One kernel per pattern: the two head kinds' bodies are specialised on their
// kind codes, and each workgroup branches once, uniformly, on its head's kind.
// M: merged heads (the epilogue carries or merges; plain patterns compile
// without those stores).
// GW: 16-row groups per wave.  GW = 2: four waves, each two groups that share
// every K and V operand read (about 120 VGPRs, four workgroups per CU).  GW =
// 1: eight waves of one group (76 VGPRs; six waves per SIMD, three workgroups
// per CU), twice the LDS reads per row but more waves to hide latency, which
// pays in launches too short to fill the GPU more than once or twice.
template <typename E, int D, int NS, int C0, int C1, bool M, int GW>
__global__ __launch_bounds__(512 / GW) __attribute__((amdgpu_waves_per_eu(GW == 1 ? 6 : 1))) void fwd_b16_kernel(
    FwdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[NS][2][TileShape<D>::BYTES];
  const PairItem item = load_uniform(&a.pairs[blockIdx.x]);
  if (item.pb < 0) return;  // schedule padding
  if (C0 == C1 || item.kind == 0)
    fwd_b16_body<E, D, NS, C0, M, GW>(a, item, ring);
  else
    fwd_b16_body<E, D, NS, C1, M, GW>(a, item, ring);
}

template <typename TE, int D>
hipError_t launch_fwd(const FwdArgs& a, int n_items, int rows_per_wave, hipStream_t stream) {
  if (n_items == 0) return hipSuccess;
  timing_begin(KID_FWD, stream);
  hipError_t err;
  if constexpr (Is16<TE>::value) {
    err = with_kind_codes(a.pattern, [&](auto c0, auto c1, auto m) {
      constexpr int C0 = decltype(c0)::value, C1 = decltype(c1)::value;
      constexpr bool M = decltype(m)::value;
      if constexpr (D <= 64) {
        if (rows_per_wave == 16) {
          hipLaunchKernelGGL((fwd_b16_kernel<TE, D, kFwdStages, C0, C1, M, 1>), dim3(n_items), dim3(512), 0, stream,
                             a);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((fwd_b16_kernel<TE, D, kFwdStages, C0, C1, M, 2>), dim3(n_items), dim3(kThreads), 0, stream,
                         a);
      return hipGetLastError();
    });
  } else {
    hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3(n_items), dim3(kThreads), 0, stream, a);
    err = hipGetLastError();
  }
  timing_end(KID_FWD, stream);
  return err;
}

template hipError_t launch_fwd<bf16, 32>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd<bf16, 64>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd<bf16, 128>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd<f16, 32>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd<f16, 64>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd<f16, 128>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd<float, 32>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd<float, 64>(const FwdArgs&, int, int, hipStream_t);
template hipError_t launch_fwd<float, 128>(const FwdArgs&, int, int, hipStream_t);

}  // namespace st
