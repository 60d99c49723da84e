// Plane-prefix scan (Fathom summary, bit-plane paragraph; per-token cost
// noted in its closing paragraph on HBM-resident scans).
//
// Score of token i under a plan (depth t_j, group query qbar):
//   s_i = sum_{t_j>0} qbar_j * (off_bj + scale_bj * (c_ij * 2^(4-t_j) + (2^(4-t_j)-1)/2))
// with c_ij the t_j-bit prefix code.  Since c * 2^(4-t) = sum_{p<t} bit_p * 2^(3-p),
// every plane bit carries a weight that does not depend on t:
//   s_i = C_b + sum_{p=0..3} 2^(3-p) * acc_p,  acc_p = sum_{j: t_j>p, bit_pij=1} qbar_j * scale_bj
//   C_b = sum_{t_j>0} qbar_j * off_bj + (qbar_j * (2^(4-t_j)-1)/2) * scale_bj
//
// Mapping onto a wave64: one wave owns a 64-token block at a time, lane l is
// token 64b+l, so the 64-bit plane word of a block IS the set of lanes whose
// bit is 1.  The word is fetched with a scalar load and used directly as a
// lane mask (inverse ballot), and the block's fp16 scale, also a scalar load,
// feeds a mixed-precision FMA (v_fma_mix_f32) without conversion.  C_b is
// computed lane-parallel over (channel slot, block) pairs and reduced with
// cross-lane shuffles.  The active channel list (sorted by depth) is built
// once per workgroup in LDS.
#include "common.hpp"

namespace sdq {

constexpr int kScanWaves = 4;
constexpr int kScanTB = 8;     // 64-token blocks per wave tile

// The index is read-only for the whole launch: reading it through the
// constant address space lets wave-uniform loads go to the scalar unit
// (s_load into SGPRs) instead of vector loads plus v_readfirstlane.
template <typename T>
using cptr = const __attribute__((address_space(4))) T*;
// The pointer is the same in every lane; readfirstlane makes that explicit
// (the compiler cannot always prove it) so the address lives in SGPRs.
template <typename T>
__device__ __forceinline__ cptr<T> as_const(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return (cptr<T>)((uint64_t(hi) << 32) | lo);
}

struct ScanCtx {
  const uint32_t* planes;
  const uint32_t* meta;
  size_t nw;          // 32-bit words per plane row (n/32)
  int nb64;
  int g;
  int A;
  const int* s_j;
  const int* s_t;
  const float* s_q;
  const float* s_qm;
};

template <int T, int TB>
__device__ __forceinline__ void accum_channel(cptr<uint64_t> prow, size_t pstride,
                                              cptr<uint32_t> mrow, float qv,
                                              float (&acc)[4][TB]) {
#pragma unroll
  for (int k = 0; k < TB; ++k) {
    const uint32_t mw = mrow[k];
    const float sc = float(__builtin_bit_cast(_Float16, uint16_t(mw & 0xFFFFu)));
#pragma unroll
    for (int p = 0; p < T; ++p) {
      const uint64_t m = prow[size_t(p) * pstride + k];
      const float upd = __builtin_fmaf(sc, qv, acc[p][k]);
      acc[p][k] = __builtin_amdgcn_inverse_ballot_w64(m) ? upd : acc[p][k];
    }
  }
}

template <int TB>
__device__ __forceinline__ void scan_tile(const ScanCtx& c, int b0, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  float acc[4][TB];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int k = 0; k < TB; ++k) acc[p][k] = 0.0f;

  const size_t pstride = c.nw / 2;   // 64-bit words per plane row
  for (int a = 0; a < c.A; ++a) {
    const int j = __builtin_amdgcn_readfirstlane(c.s_j[a]);
    const int t = __builtin_amdgcn_readfirstlane(c.s_t[a]);
    const float qv = c.s_q[a];
    const size_t row = size_t(c.g) * kHeadDim + j;
    cptr<uint32_t> mrow = as_const(c.meta + row * c.nb64 + b0);
    cptr<uint64_t> prow =
        as_const(reinterpret_cast<const uint64_t*>(c.planes + row * 4 * c.nw) + b0);
    switch (t) {
      case 4: accum_channel<4, TB>(prow, pstride, mrow, qv, acc); break;
      case 3: accum_channel<3, TB>(prow, pstride, mrow, qv, acc); break;
      case 2: accum_channel<2, TB>(prow, pstride, mrow, qv, acc); break;
      default: accum_channel<1, TB>(prow, pstride, mrow, qv, acc); break;
    }
  }

  // constant term per block, lane-parallel: lane = (channel slot, block)
  constexpr int SLOTS = 64 / TB;
  const int slot = lane / TB, kb = lane % TB;
  float cacc = 0.0f;
  for (int a0 = 0; a0 < c.A; a0 += SLOTS) {
    const int a = a0 + slot;
    if (a < c.A) {
      const int j = c.s_j[a];
      const uint32_t mw = c.meta[(size_t(c.g) * kHeadDim + j) * c.nb64 + b0 + kb];
      const float off = float(__builtin_bit_cast(_Float16, uint16_t(mw >> 16)));
      const float sc = float(__builtin_bit_cast(_Float16, uint16_t(mw & 0xFFFFu)));
      cacc = __builtin_fmaf(off, c.s_q[a], cacc);
      cacc = __builtin_fmaf(sc, c.s_qm[a], cacc);
    }
  }
#pragma unroll
  for (int m = TB; m < 64; m <<= 1) cacc += __shfl_xor(cacc, m, 64);

#pragma unroll
  for (int k = 0; k < TB; ++k) {
    const float ck = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cacc), k));
    const float s = ((acc[0][k] * 8.0f + acc[1][k] * 4.0f) + acc[2][k] * 2.0f) + acc[3][k];
    out[size_t(b0 + k) * 64 + lane] = s + ck;
  }
}

__global__ __launch_bounds__(kScanWaves * 64) void fathom_scan_kernel(
    const uint32_t* __restrict__ planes, const uint32_t* __restrict__ meta,
    const uint8_t* __restrict__ depth, const float* __restrict__ qbar, int n, int nb64,
    float* __restrict__ scores) {
  __shared__ int s_j[kHeadDim];
  __shared__ int s_t[kHeadDim];
  __shared__ float s_q[kHeadDim];
  __shared__ float s_qm[kHeadDim];
  __shared__ int s_A;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  if (wave == 0) {
    // active channels sorted by depth (4 first); depths outside 1..4 are unread
    const int t0 = depth[size_t(g) * kHeadDim + lane];
    const int t1 = depth[size_t(g) * kHeadDim + lane + 64];
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
    for (int L = 4; L >= 1; --L) {
      const uint64_t b0 = __ballot(t0 == L), b1 = __ballot(t1 == L);
      if (t0 == L) {
        const int pos = base + __popcll(b0 & lt);
        s_j[pos] = lane;
        s_t[pos] = L;
      }
      if (t1 == L) {
        const int pos = base + __popcll(b0) + __popcll(b1 & lt);
        s_j[pos] = lane + 64;
        s_t[pos] = L;
      }
      base += __popcll(b0) + __popcll(b1);
    }
    if (lane == 0) s_A = base;
  }
  __syncthreads();
  const int A = __builtin_amdgcn_readfirstlane(s_A);
  if (tid < A) {
    const int j = s_j[tid];
    const float qv = qbar[size_t(g) * kHeadDim + j];
    const float half_gap = float((1 << (4 - s_t[tid])) - 1) * 0.5f;
    s_q[tid] = qv;
    s_qm[tid] = qv * half_gap;
  }
  __syncthreads();

  ScanCtx c{planes, meta, size_t(n) / 32, nb64, g, A, s_j, s_t, s_q, s_qm};
  float* out = scores + size_t(g) * n;
  // wave index is uniform within a wave; say so, so that tile addresses stay scalar
  const int b0 = __builtin_amdgcn_readfirstlane((blockIdx.x * kScanWaves + wave) * kScanTB);
  if (b0 >= nb64) return;
  if (b0 + kScanTB <= nb64) {
    scan_tile<kScanTB>(c, b0, out);
  } else {
    for (int b = b0; b < nb64; ++b) scan_tile<1>(c, b, out);
  }
}

}  // namespace sdq

using namespace sdq;

extern "C" int fathom_scan(const uint32_t* planes, const uint32_t* meta, const uint8_t* depth,
                           const float* qbar, int G, int d, int n, float* scores,
                           hipStream_t stream) {
  SDQ_REQUIRE(planes && meta && depth && qbar && scores, "fathom_scan: null pointer");
  SDQ_REQUIRE(G >= 1, "fathom_scan: G=%d must be >= 1", G);
  SDQ_REQUIRE(n >= 64 && n % 64 == 0, "fathom_scan: n=%d must be a positive multiple of 64", n);
  SDQ_REQUIRE(d == kHeadDim, "fathom_scan: d=%d unsupported (only 128)", d);
  const int nb64 = n / 64;
  dim3 grid(cdiv(nb64, kScanWaves * kScanTB), G);
  hipLaunchKernelGGL(fathom_scan_kernel, grid, dim3(kScanWaves * 64), 0, stream, planes, meta,
                     depth, qbar, n, nb64, scores);
  return check_launch("fathom_scan");
}
