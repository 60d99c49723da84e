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
                                              int budget) {
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

  uint32_t T = 0;
  if (K > 0) {
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int t = 0; t < NT; ++t) cnt += wave_count(v0[t] >= cand) + wave_count(v1[t] >= cand);
      if (cnt >= K) T = cand;
    }
  }
  int gt = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) gt += wave_count(v0[t] > T) + wave_count(v1[t] > T);
  const int rem = K - gt;                  // bits to take among those equal to T

  const uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));
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
