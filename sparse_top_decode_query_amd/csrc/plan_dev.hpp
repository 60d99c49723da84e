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
// T's exponent field comes from a 256-bin histogram of the candidates'
// exponent fields in LDS and one wave scan over it (the largest exponent e
// with at least K candidates at or above it).  When that exponent is not 0,
// the candidates sharing it hold at most one bit per channel (a channel's
// normal gains are 2 binades apart), so at most 128 of them exist: they are
// compacted into LDS and T is the one whose rank among them is the one still
// needed, found by counting instead of 23 dependent search steps.  A zero
// exponent (subnormal gains, or infinite ones) takes the bitwise search over
// the mantissa instead.  `lds` is 384 words private to the wave.
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
  // w = (qbar*qbar)*var as two rounded multiplies.  A variance is never
  // negative: a weight that is negative, -0 or NaN (a bad variance handed in)
  // is read as +0, so every gain's exponent field indexes the 256-bin
  // histogram below.
  float w0 = __fmul_rn(__fmul_rn(a0, a0), va0);
  float w1 = __fmul_rn(__fmul_rn(a1, a1), va1);
  w0 = w0 > 0.0f ? w0 : 0.0f;
  w1 = w1 > 0.0f ? w1 : 0.0f;

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
  auto lds_sync = [] {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (K > 0) {
    // exponent field of T from a histogram of the candidates' exponent fields
    uint32_t* hist = lds + kHeadDim;                 // 256 bins after the bucket
    reinterpret_cast<uint4*>(hist)[l] = make_uint4(0u, 0u, 0u, 0u);
    lds_sync();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      atomicAdd(&hist[v0[t] >> 23], 1u);
      atomicAdd(&hist[v1[t] >> 23], 1u);
    }
    lds_sync();
    const uint4 c4 = reinterpret_cast<const uint4*>(hist)[l];     // bins 4l .. 4l+3
    const int s4 = int(c4.x + c4.y + c4.z + c4.w);
    const int inc = wave_incl_scan(s4);
    const int ge3 = wave_last(inc) - inc + int(c4.w);             // candidates with exponent >= 4l+3
    const int ge2 = ge3 + int(c4.z), ge1 = ge2 + int(c4.y), ge0 = ge1 + int(c4.x);
    // the largest e with ge(e) >= K: ge falls as e rises, so the lanes with
    // such a bin are a prefix of the wave and e is the top one of the last
    const int eb = ge3 >= K ? 3 : (ge2 >= K ? 2 : (ge1 >= K ? 1 : (ge0 >= K ? 0 : -1)));
    const int abv = eb == 3 ? ge3 - int(c4.w) : (eb == 2 ? ge3 : (eb == 1 ? ge2 : ge1));
    const uint64_t own = __ballot(eb >= 0);
    const int src_lane = 63 - __builtin_clzll(own);
    const uint32_t e = uint32_t(__builtin_amdgcn_readlane(4 * l + eb, src_lane));
    const int above = __builtin_amdgcn_readlane(abv, src_lane);  // candidates with exponent > e
    T = e << 23;
    lds_sync();
    if (e == 0 || e == 255) {                       // subnormal or infinite gains
      search(22, 0);
    } else {
      // the bucket: candidates with T's exponent; r = rank of T within it
      uint32_t u0 = 0, u1 = 0;
      bool h0 = false, h1 = false;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if ((v0[t] >> 23) == e) { u0 = v0[t]; h0 = true; }
        if ((v1[t] >> 23) == e) { u1 = v1[t]; h1 = true; }
      }
      const int r = K - above;
      const uint64_t b0 = __ballot(h0), b1 = __ballot(h1);
      const int m0 = __popcll(b0), m = m0 + __popcll(b1);
      if (h0) lds[__popcll(b0 & lt)] = u0;
      if (h1) lds[m0 + __popcll(b1 & lt)] = u1;
      // pad to a multiple of 8 with zeros (below every bucket value, so they
      // count nowhere) and read 8 values per round, loads ahead of compares
      const int m8 = (m + 7) & ~7;
      if (l < m8 - m) lds[m + l] = 0u;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint4* l4 = reinterpret_cast<const uint4*>(lds);
      if (m <= 64) {
        // one bucket value a lane (the usual case: 14-26 values at B = 56)
        const uint32_t x = lds[l];
        int gt = 0, ge = 0;
        for (int i = 0; i < m8 / 4; i += 2) {
          const uint4 xa = l4[i], xb = l4[i + 1];
          const uint32_t xs[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            gt += xs[k] > x;
            ge += xs[k] >= x;
          }
        }
        const uint64_t c = __ballot(l < m && gt < r && r <= ge);
        T = uint32_t(__builtin_amdgcn_readlane(int(x), int(__builtin_ctzll(c))));
      } else {
        int gt0 = 0, ge0 = 0, gt1 = 0, ge1 = 0;
        for (int i = 0; i < m8 / 4; i += 2) {
          const uint4 xa = l4[i], xb = l4[i + 1];
          const uint32_t xs[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            gt0 += xs[k] > u0;
            ge0 += xs[k] >= u0;
            gt1 += xs[k] > u1;
            ge1 += xs[k] >= u1;
          }
        }
        const uint64_t c0 = __ballot(h0 && gt0 < r && r <= ge0);
        const uint64_t c1 = __ballot(h1 && gt1 < r && r <= ge1);
        T = c0 ? uint32_t(__builtin_amdgcn_readlane(int(u0), int(__builtin_ctzll(c0))))
               : uint32_t(__builtin_amdgcn_readlane(int(u1), int(__builtin_ctzll(c1))));
      }
      __builtin_amdgcn_wave_barrier();              // lds is free again
    }
  }
  // Bits above T, and the bits equal to T in (j, t) order, counted with one
  // packed wave scan: per lane (#gain > T) | (#gain == T of channel l) << 10
  // | (#gain == T of channel l+64) << 20, each field below 2^10.
  int cg = 0, ce0 = 0, ce1 = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    cg += int(v0[t] > T) + int(v1[t] > T);
    ce0 += int(v0[t] == T);
    ce1 += int(v1[t] == T);
  }
  const int packed = K > 0 ? (cg | ce0 << 10 | ce1 << 20) : 0;
  const int inc = wave_incl_scan(packed);
  const int tot = wave_last(inc);
  const int excl = inc - packed;
  const int gt = tot & 0x3FF;
  const int rem = K - gt;                  // bits to take among those equal to T
  const int before0 = (excl >> 10) & 0x3FF;
  const int before1 = ((tot >> 10) & 0x3FF) + ((excl >> 20) & 0x3FF);

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
