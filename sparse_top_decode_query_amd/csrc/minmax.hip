// Block scores against per-block min/max key summaries (OasisKV review,
// Quest-style summaries in the background section; per-KV-head ranking in
// the core-method section).
//
// For one head, max(q*mn, q*mx) is q*mx when q >= 0 and q*mn otherwise, so
// with P_j = sum_h max(q_hj, 0) and N_j = sum_h min(q_hj, 0) over the group's
// heads, the group score is
//   S_b = sum_j P_j * mx_bj + N_j * mn_bj
// -- two fused multiply-adds per dimension per block, whatever the group size.
// The fp16 summaries feed v_fma_mix_f32 directly.  16 lanes share a block
// (8 dimensions each, one 16-byte load of mn and one of mx), a wave covers 4
// blocks per step; the 16 partial sums are reduced with DPP row operations.
// HBM-bound: 512 bytes of summaries per block of 16 tokens.
#include "common.hpp"

namespace sdq {

constexpr int kMmThreads = 256;
constexpr int kMmBlocksPerIter = kMmThreads / 16;   // 16 blocks per workgroup step
constexpr int kMmIters = 8;                          // steps per workgroup

__device__ __forceinline__ float fma_h(uint32_t w, int hi, float a, float acc) {
  const uint16_t bits = hi ? uint16_t(w >> 16) : uint16_t(w & 0xFFFFu);
  return __builtin_fmaf(float(__builtin_bit_cast(_Float16, bits)), a, acc);
}

__global__ __launch_bounds__(kMmThreads) void minmax_block_scan_kernel(
    const uint4* __restrict__ bmin, const uint4* __restrict__ bmax, const float* __restrict__ q,
    int Hgrp, int nb, int nb_cap, float* __restrict__ S) {
  const int rg = blockIdx.y;
  const int tid = threadIdx.x;
  const int sub = tid & 15;             // which 8 dimensions
  const int slot = tid >> 4;            // which block of the step
  float P[8], N[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    P[e] = 0.0f;
    N[e] = 0.0f;
  }
  const float* qg = q + size_t(rg) * Hgrp * kHeadDim + sub * 8;
  for (int h = 0; h < Hgrp; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = qg[size_t(h) * kHeadDim + e];
      P[e] += fmaxf(v, 0.0f);
      N[e] += fminf(v, 0.0f);
    }
  }
  const size_t row = size_t(rg) * nb_cap;          // summaries; scores rows are nb long
  // every step's summaries are requested before the first is used (the
  // index is clamped so the loads stay unconditional and in bounds)
  uint4 lo[kMmIters], hi[kMmIters];
#pragma unroll
  for (int it = 0; it < kMmIters; ++it) {
    const int b = (blockIdx.x * kMmIters + it) * kMmBlocksPerIter + slot;
    const int bc = b < nb ? b : nb - 1;
    lo[it] = bmin[(row + bc) * 16 + sub];
    hi[it] = bmax[(row + bc) * 16 + sub];
  }
#pragma unroll
  for (int it = 0; it < kMmIters; ++it) {
    const int b = (blockIdx.x * kMmIters + it) * kMmBlocksPerIter + slot;
    const uint32_t lw[4] = {lo[it].x, lo[it].y, lo[it].z, lo[it].w};
    const uint32_t hw[4] = {hi[it].x, hi[it].y, hi[it].z, hi[it].w};
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fma_h(hw[e], 0, P[2 * e], acc);
      acc = fma_h(hw[e], 1, P[2 * e + 1], acc);
      acc = fma_h(lw[e], 0, N[2 * e], acc);
      acc = fma_h(lw[e], 1, N[2 * e + 1], acc);
    }
    acc = row16_sum(acc);                      // the block's 16 lanes form one DPP row
    if (sub == 0 && b < nb) S[size_t(rg) * nb + b] = acc;
  }
}

}  // namespace sdq

using namespace sdq;

extern "C" int minmax_block_scan(const uint16_t* bmin, const uint16_t* bmax, const float* q,
                                 int RG, int H_grp, int nb, int nb_cap, int d,
                                 float* block_scores, hipStream_t stream) {
  SDQ_REQUIRE(bmin && bmax && q && block_scores, "minmax_block_scan: null pointer");
  SDQ_REQUIRE(RG >= 1 && H_grp >= 1 && nb >= 1, "minmax_block_scan: RG=%d, H_grp=%d, nb=%d must be >= 1",
              RG, H_grp, nb);
  SDQ_REQUIRE(nb <= nb_cap, "minmax_block_scan: nb=%d exceeds nb_cap=%d", nb, nb_cap);
  SDQ_REQUIRE(d == kHeadDim, "minmax_block_scan: d=%d unsupported (only 128)", d);
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(bmin) % 16 == 0 && reinterpret_cast<uintptr_t>(bmax) % 16 == 0,
              "minmax_block_scan: summaries must be 16-byte aligned");
  dim3 grid(cdiv(nb, kMmIters * kMmBlocksPerIter), RG);
  hipLaunchKernelGGL(minmax_block_scan_kernel, grid, dim3(kMmThreads), 0, stream,
                     reinterpret_cast<const uint4*>(bmin), reinterpret_cast<const uint4*>(bmax), q,
                     H_grp, nb, nb_cap, block_scores);
  return check_launch("minmax_block_scan");
}
