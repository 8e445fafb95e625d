// Fused sparse attention forward for gfx950.
//
// Computes, per head, out_t = softmax_{j in S(t)}(q_t . k_j / sqrt(D)) v_j and
// lse_t (nlp-lineage, "The notation"; llm-arch-kb "Sparse Transformer", §2,
// masked logits carry no mass).  Only the block pairs the LUT lists are
// visited (llm-arch-kb §2 "Per-layer cost": a block-sparse product, not a
// masked dense one); inside PARTIAL blocks each logit outside the row's key
// run is set to -inf, and 16-key sub-blocks that no row of a wave needs are
// skipped.
//
// Work item = (row block of 64 kernel rows, batch*head).  4 waves, each owns
// 16 rows.  Per key block: K (row-major) and V (transposed for bf16, so the
// P.V operand is a contiguous LDS read) are staged in LDS; S^T = K Q^T runs on
// MFMA so each lane holds 16 logits of its own query; the online softmax keeps
// the running max / sum in registers (cross-lane only over the 4 lanes of a
// query); O^T += V^T P^T runs on MFMA with P packed to bf16 in registers.
#include "st_device.hpp"
#include "st_kernels.hpp"

namespace st {

namespace {

template <typename TE, int D>
struct FwdLds {
  static constexpr bool BF = IsBf16<TE>::value;
  static constexpr int KP = BF ? D + 8 : D + 2;        // K row pitch (elements)
  static constexpr int VP = BF ? kBlock + 8 : D + 2;   // bf16: V^T [D][VP]; fp32: V [64][VP]
  static constexpr int K_ELEMS = kBlock * KP;
  static constexpr int V_ELEMS = BF ? D * VP : kBlock * VP;
};

// Stage key block kb of K and V into LDS (zeros for padding keys).
template <typename TE, int D>
__device__ __forceinline__ void stage_kv(const TE* __restrict__ K, const TE* __restrict__ V,
                                         const Geometry& g, int kb, TE* Ks, TE* Vs) {
  using L = FwdLds<TE, D>;
  const int tid = threadIdx.x;
  if constexpr (L::BF) {
    // unit = (key pair, 8-element chunk); the pair lets V^T be written in 32-bit words
    constexpr int CH = D / 8;
    for (int u = tid; u < (kBlock / 2) * CH; u += kThreads) {
      const int pr = u / CH, ch = u - pr * CH;
      const int K0 = kb * kBlock + 2 * pr;
      const int p0 = key_position(g, K0), p1 = key_position(g, K0 + 1);
      uint4 k0 = {0, 0, 0, 0}, k1 = {0, 0, 0, 0}, v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
      if (p0 >= 0) {
        k0 = *(const uint4*)(K + (size_t)p0 * D + ch * 8);
        v0 = *(const uint4*)(V + (size_t)p0 * D + ch * 8);
      }
      if (p1 >= 0) {
        k1 = *(const uint4*)(K + (size_t)p1 * D + ch * 8);
        v1 = *(const uint4*)(V + (size_t)p1 * D + ch * 8);
      }
      *(uint4*)(Ks + (2 * pr) * L::KP + ch * 8) = k0;
      *(uint4*)(Ks + (2 * pr + 1) * L::KP + ch * 8) = k1;
      const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w};
      const uint32_t b[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // elements 2w (low half) and 2w+1 (high half) of each row
        const uint32_t lo = (a[w] & 0xffffu) | (b[w] << 16);
        const uint32_t hi = (a[w] >> 16) | (b[w] & 0xffff0000u);
        *(uint32_t*)(Vs + (ch * 8 + 2 * w) * L::VP + 2 * pr) = lo;
        *(uint32_t*)(Vs + (ch * 8 + 2 * w + 1) * L::VP + 2 * pr) = hi;
      }
    }
  } else {
    constexpr int CH = D / 4;
    for (int u = tid; u < kBlock * CH; u += kThreads) {
      const int r = u / CH, ch = u - r * CH;
      const int p = key_position(g, kb * kBlock + r);
      float4 kk = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (p >= 0) {
        kk = *(const float4*)(K + (size_t)p * D + ch * 4);
        vv = *(const float4*)(V + (size_t)p * D + ch * 4);
      }
      float* kd = (float*)Ks + r * L::KP + ch * 4;
      float* vd = (float*)Vs + r * L::VP + ch * 4;
      *(float2*)kd = make_float2(kk.x, kk.y);
      *(float2*)(kd + 2) = make_float2(kk.z, kk.w);
      *(float2*)vd = make_float2(vv.x, vv.y);
      *(float2*)(vd + 2) = make_float2(vv.z, vv.w);
    }
  }
}

template <typename TE, int D>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdArgs a) {
  using L = FwdLds<TE, D>;
  constexpr bool BF = L::BF;
  constexpr int NQ = BF ? D / 32 : D / 4;  // Q operand registers (MFMA k-steps over D)
  constexpr int ND = D / 16;               // 16-wide output column blocks
  __shared__ __attribute__((aligned(16))) TE Ks[L::K_ELEMS];
  __shared__ __attribute__((aligned(16))) TE Vs[L::V_ELEMS];

  const int2 item = a.items[blockIdx.x];
  const int qb = item.x, bh = item.y;
  const int h = bh % a.H;
  const KindDev kd = a.kinds[h & 1];
  const Geometry& g = kd.geo;
  const size_t base = (size_t)bh * a.T * D;
  const TE* __restrict__ Q = (const TE*)a.q + base;
  const TE* __restrict__ Kg = (const TE*)a.k + base;
  const TE* __restrict__ Vg = (const TE*)a.v + base;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int R = qb * kBlock + wave * 16 + li;
  const int t = row_position(g, R);
  int lo = 1, hi = 0;
  if (t >= 0) row_interval(g, R, t, lo, hi);
  const int wlo = wave_min(lo <= hi ? lo : 0x7fffffff);
  const int whi = wave_max(lo <= hi ? hi : -1);
  const bool wave_active = whi >= 0;

  // Q operand (B of S^T = K Q^T): lane holds Q[t][kw*lg + ...] of each k-step.
  typedef typename std::conditional<BF, bf16x8, float>::type QOp;
  QOp qop[NQ];
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    if constexpr (BF) {
      uint4 raw = {0, 0, 0, 0};
      if (t >= 0) raw = *(const uint4*)(Q + (size_t)t * D + 32 * s + 8 * lg);
      qop[s] = __builtin_bit_cast(bf16x8, raw);
    } else {
      qop[s] = (t >= 0) ? (float)Q[(size_t)t * D + 4 * s + lg] : 0.f;
    }
  }

  f32x4 acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.sl2;

  const int e0 = kd.row_ptr[qb], e1 = kd.row_ptr[qb + 1];
  for (int e = e0; e < e1; ++e) {
    const int kb = kd.col_idx[e];
    const bool full = kd.flags[e] != 0;
    __syncthreads();
    stage_kv<TE, D>(Kg, Vg, g, kb, Ks, Vs);
    __syncthreads();
    if (!wave_active) continue;

    const int k0 = kb * kBlock;
    bool need[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      need[b] = full || (k0 + 16 * b <= whi && k0 + 16 * b + 15 >= wlo);

    // S^T = K Q^T, one 16x16 block per 16 keys
    f32x4 s[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      s[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (!need[b]) continue;
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        if constexpr (BF) {
          const bf16x8 av = *(const bf16x8*)(Ks + (16 * b + li) * L::KP + 32 * k + 8 * lg);
          s[b] = mfma_bf16(av, qop[k], s[b]);
        } else {
          const float av = ((const float*)Ks)[(16 * b + li) * L::KP + 4 * k + lg];
          s[b] = mfma_f32(av, qop[k], s[b]);
        }
      }
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
    const float mb = (m_new == -INFINITY) ? 0.f : m_new * sl2;
    const float alpha = fast_exp2(m_run * sl2 - mb);
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(fmaf(s[b][i], sl2, -mb));
        s[b][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] *= alpha;

    // O^T += V^T P^T
    if constexpr (BF) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (!need[2 * kk] && !need[2 * kk + 1]) continue;
        const bf16x8 pb = pack_b_operand(s[2 * kk], s[2 * kk + 1]);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const TE* row = Vs + (16 * d + li) * L::VP + 32 * kk + 4 * lg;
          const bf16x8 av = concat(*(const bf16x4*)row, *(const bf16x4*)(row + 16));
          acc[d] = mfma_bf16(av, pb, acc[d]);
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (!need[b]) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const float av = ((const float*)Vs)[(16 * b + 4 * lg + i) * L::VP + 16 * d + li];
            acc[d] = mfma_f32(av, s[b][i], acc[d]);
          }
        }
      }
    }
  }

  // epilogue: normalise, write O (bf16 RNE or fp32) and lse (natural log)
  const float lsum = group4_sum(l_run);
  if (t < 0) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  TE* O = (TE*)a.o + base + (size_t)t * D;
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const f32x4 o = acc[d] * inv;
    if constexpr (BF) {
      *(bf16x4*)(O + 16 * d + 4 * lg) = to_bf16x4(o);
    } else {
      *(float4*)(O + 16 * d + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
  if (lg == 0)
    a.lse[(size_t)bh * a.T + t] = lsum > 0.f ? (m_run * sl2 + fast_log2(lsum)) * kLn2 : -INFINITY;
}

}  // namespace

template <typename TE, int D>
hipError_t launch_fwd(const FwdArgs& a, int n_items, hipStream_t stream) {
  if (n_items == 0) return hipSuccess;
  timing_begin(KID_FWD, stream);
  hipLaunchKernelGGL((fwd_kernel<TE, D>), dim3(n_items), dim3(kThreads), 0, stream, a);
  const hipError_t err = hipGetLastError();
  timing_end(KID_FWD, stream);
  return err;
}

template hipError_t launch_fwd<bf16, 32>(const FwdArgs&, int, hipStream_t);
template hipError_t launch_fwd<bf16, 64>(const FwdArgs&, int, hipStream_t);
template hipError_t launch_fwd<float, 32>(const FwdArgs&, int, hipStream_t);
template hipError_t launch_fwd<float, 64>(const FwdArgs&, int, hipStream_t);

}  // namespace st
