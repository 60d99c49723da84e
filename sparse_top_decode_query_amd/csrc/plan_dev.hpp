// The per-KV-head read plan as a device function of one wavefront (Fathom
// summary, water-filling paragraph), shared by the plan kernel and by the
// fused plan + scan kernel so that both give the identical plan.
//
// The 4d candidate bits (channel j, bit t) have gain v(j,t) = w_j * 4^-t with
// w_j = (qbar_j * qbar_j) * var_j, qbar the float32 sum of the group's query
// rows in head order.  The plan takes the first min(B, 4d) bits in the order
// (gain desc, j asc, t asc).  Lane l owns channels l and l+64 (8 candidate
// bits); the B-th largest gain T is found by a 31-step bitwise search over the
// gains' bit patterns (non-negative floats order like their bit patterns),
// counting candidates with wave ballots.  Bits with gain > T are taken, and of
// the bits with gain == T the first B - #(gain > T) in (j, t) order.  The
// uniform baseline plan takes the n_channels channels of largest w_j (ties to
// the lower channel), each at depth 4.
//
// The search first fixes T's exponent field (8 steps).  When that exponent is
// not 0, the candidates sharing it hold at most one bit per channel (a
// channel's normal gains are 2 binades apart), so at most 128 of them exist:
// they are compacted into `lds` (128 words, private to the wave) and T is the
// one whose rank among them is the one still needed, found by counting
// instead of 23 more dependent search steps.  A zero exponent (subnormal
// gains, or infinite ones) continues the bitwise search instead.
#pragma once
#include "common.hpp"

namespace sdq {

__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

struct HeadPlan {
  int d0, d1;        // depth of channels lane and lane + 64
  float a0, a1;      // qbar of channels lane and lane + 64
};

// Whole wavefront (64 lanes) of one KV head g.
template <bool UNIFORM>
__device__ __forceinline__ HeadPlan plan_head(const float* __restrict__ q,
                                              const float* __restrict__ var, int g, int Hgrp,
                                              int budget, uint32_t* lds) {
  const int l = threadIdx.x & 63;
  const int j0 = l, j1 = l + 64;
  const float* qg = q + size_t(g) * Hgrp * kHeadDim;
  // every load is issued before the first add (one memory round trip for
  // groups of up to kBatch heads), then the rows are summed in head order
  constexpr int kBatch = 8;
  const float va0 = var[size_t(g) * kHeadDim + j0], va1 = var[size_t(g) * kHeadDim + j1];
  float a0 = 0.0f, a1 = 0.0f;
  for (int h0 = 0; h0 < Hgrp; h0 += kBatch) {
    float r0[kBatch], r1[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int h = h0 + k < Hgrp ? h0 + k : Hgrp - 1;
      r0[k] = qg[size_t(h) * kHeadDim + j0];
      r1[k] = qg[size_t(h) * kHeadDim + j1];
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {              // branch-free: rows past Hgrp are skipped
      const bool in = h0 + k < Hgrp;
      const float s0 = __fadd_rn(a0, r0[k]), s1 = __fadd_rn(a1, r1[k]);
      a0 = h0 + k == 0 ? r0[k] : (in ? s0 : a0);
      a1 = h0 + k == 0 ? r1[k] : (in ? s1 : a1);
    }
  }
  // w = (qbar*qbar)*var as two rounded multiplies; -0 folded onto +0
  const float w0 = __fadd_rn(__fmul_rn(__fmul_rn(a0, a0), va0), 0.0f);
  const float w1 = __fadd_rn(__fmul_rn(__fmul_rn(a1, a1), va1), 0.0f);

  constexpr int NT = UNIFORM ? 1 : 4;      // candidate bits per channel
  const float step[4] = {1.0f, 0.25f, 0.0625f, 0.015625f};
  uint32_t v0[NT], v1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    v0[t] = __float_as_uint(__fmul_rn(w0, step[t]));
    v1[t] = __float_as_uint(__fmul_rn(w1, step[t]));
  }
  const int total = NT * kHeadDim;
  const int K = budget < total ? budget : total;

  const uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));
  uint32_t T = 0;
  auto search = [&](int hi, int lo) {
    for (int bit = hi; bit >= lo; --bit) {
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int t = 0; t < NT; ++t) cnt += wave_count(v0[t] >= cand) + wave_count(v1[t] >= cand);
      if (cnt >= K) T = cand;
    }
  };
  if (K > 0) {
    search(30, 23);                                  // exponent field of T
    const uint32_t e = T >> 23;
    if (e == 0 || e == 255) {                       // subnormal or infinite gains
      search(22, 0);
    } else {
      // the bucket: candidates with T's exponent; r = rank of T within it
      const uint32_t above_cut = (e + 1) << 23;
      int above = 0;
      uint32_t u0 = 0, u1 = 0;
      bool h0 = false, h1 = false;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        above += wave_count(v0[t] >= above_cut) + wave_count(v1[t] >= above_cut);
        if ((v0[t] >> 23) == e) { u0 = v0[t]; h0 = true; }
        if ((v1[t] >> 23) == e) { u1 = v1[t]; h1 = true; }
      }
      const int r = K - above;
      const uint64_t b0 = __ballot(h0), b1 = __ballot(h1);
      const int m0 = __popcll(b0), m = m0 + __popcll(b1);
      if (h0) lds[__popcll(b0 & lt)] = u0;
      if (h1) lds[m0 + __popcll(b1 & lt)] = u1;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      int gt0 = 0, ge0 = 0, gt1 = 0, ge1 = 0;
      for (int i = 0; i < m; ++i) {
        const uint32_t x = lds[i];
        gt0 += x > u0;
        ge0 += x >= u0;
        gt1 += x > u1;
        ge1 += x >= u1;
      }
      const uint64_t c0 = __ballot(h0 && gt0 < r && r <= ge0);
      const uint64_t c1 = __ballot(h1 && gt1 < r && r <= ge1);
      T = c0 ? uint32_t(__builtin_amdgcn_readlane(int(u0), int(__builtin_ctzll(c0))))
             : uint32_t(__builtin_amdgcn_readlane(int(u1), int(__builtin_ctzll(c1))));
      __builtin_amdgcn_wave_barrier();              // lds is free again
    }
  }
  int gt = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) gt += wave_count(v0[t] > T) + wave_count(v1[t] > T);
  const int rem = K - gt;                  // bits to take among those equal to T

  int before0 = 0, total0 = 0, before1 = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint64_t e0 = __ballot(K > 0 && v0[t] == T);
    before0 += __popcll(e0 & lt);
    total0 += __popcll(e0);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) before1 += __popcll(__ballot(K > 0 && v1[t] == T) & lt);
  before1 += total0;

  int d0 = 0, d1 = 0, r0 = before0, r1 = before1;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const bool eq0 = K > 0 && v0[t] == T, eq1 = K > 0 && v1[t] == T;
    d0 += (K > 0 && v0[t] > T) || (eq0 && r0 < rem);
    d1 += (K > 0 && v1[t] > T) || (eq1 && r1 < rem);
    r0 += eq0;
    r1 += eq1;
  }
  if (UNIFORM) {
    d0 *= 4;
    d1 *= 4;
  }
  return HeadPlan{d0, d1, a0, a1};
}

}  // namespace sdq
