// Index construction from the bf16 key cache:
//  * fathom_ingest: per-channel 4-bit block quantiser and channel-major bit
//    planes (Fathom summary, bit-plane paragraph);
//  * minmax_summarize: per-block min/max key summaries (OasisKV review,
//    Quest-style block summaries).
// Both run once per cached block, before any decode step; they are not part
// of the timed decode path.
#include "common.hpp"

namespace sdq {

// One thread owns a pair of adjacent channels; the 64 threads of a wave cover
// the 128 channels, so each token row (256 bytes) is read by one coalesced
// 4-byte-per-lane load.  A workgroup walks `bpw` consecutive 64-token blocks.

__global__ __launch_bounds__(64) void fathom_ingest_kernel(const uint32_t* __restrict__ keys,
                                                           int n, int nb64, int bpw,
                                                           uint32_t* __restrict__ planes,
                                                           uint32_t* __restrict__ meta) {
  const int g = blockIdx.y;
  const int pair = threadIdx.x;
  const size_t nw = size_t(n) / 32;                       // 32-token words per plane row
  for (int bb = 0; bb < bpw; ++bb) {
    const int b = blockIdx.x * bpw + bb;
    if (b >= nb64) break;
    const uint32_t* src = keys + (size_t(g) * n + size_t(b) * 64) * (kHeadDim / 2) + pair;
    uint32_t w[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) w[i] = src[size_t(i) * (kHeadDim / 2)];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float x = half ? bf16_hi(w[i]) : bf16_lo(w[i]);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
      const _Float16 off16 = _Float16(mn);
      const _Float16 sc16 = _Float16(__fdiv_rn(mx - mn, 15.0f));
      const float off = float(off16);
      const float sc = float(sc16);
      uint32_t pl[4][2] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float x = half ? bf16_hi(w[i]) : bf16_lo(w[i]);
        float r = (sc == 0.0f) ? 0.0f : rintf(__fdiv_rn(x - off, sc));
        r = fminf(fmaxf(r, 0.0f), 15.0f);
        const uint32_t code = uint32_t(r);
#pragma unroll
        for (int p = 0; p < 4; ++p) pl[p][i >> 5] |= ((code >> (3 - p)) & 1u) << (i & 31);
      }
      const int j = 2 * pair + half;
      uint32_t* prow = planes + (size_t(g) * kHeadDim + j) * 4 * nw;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        prow[size_t(p) * nw + 2 * size_t(b)] = pl[p][0];
        prow[size_t(p) * nw + 2 * size_t(b) + 1] = pl[p][1];
      }
      meta[(size_t(g) * kHeadDim + j) * nb64 + b] =
          uint32_t(__builtin_bit_cast(uint16_t, sc16)) |
          (uint32_t(__builtin_bit_cast(uint16_t, off16)) << 16);
    }
  }
}

__device__ __forceinline__ uint32_t f16_next_down(uint32_t h) {
  if (h == 0x0000u) return 0x8001u;
  return (h & 0x8000u) ? h + 1u : h - 1u;
}
__device__ __forceinline__ uint32_t f16_next_up(uint32_t h) {
  if (h == 0x8000u) return 0x0001u;
  return (h & 0x8000u) ? h - 1u : h + 1u;
}
// fp16 rounding towards -inf / +inf: round to nearest, then step one ulp
// outwards if the nearest value landed on the wrong side.
__device__ __forceinline__ uint32_t f16_round_down(float x) {
  uint32_t h = f32_to_half_bits_rne(x);
  return half_bits_to_f32(h) > x ? f16_next_down(h) : h;
}
__device__ __forceinline__ uint32_t f16_round_up(float x) {
  uint32_t h = f32_to_half_bits_rne(x);
  return half_bits_to_f32(h) < x ? f16_next_up(h) : h;
}

// One thread per adjacent channel pair; a workgroup walks `bpw` blocks.
__global__ __launch_bounds__(64) void minmax_summarize_kernel(const uint32_t* __restrict__ keys,
                                                              int n, int block, int nb, int bpw,
                                                              uint32_t* __restrict__ bmin,
                                                              uint32_t* __restrict__ bmax) {
  const int rg = blockIdx.y;
  const int pair = threadIdx.x;
  for (int bb = 0; bb < bpw; ++bb) {
    const int b = blockIdx.x * bpw + bb;
    if (b >= nb) break;
    const uint32_t* src = keys + (size_t(rg) * n + size_t(b) * block) * (kHeadDim / 2) + pair;
    float lo0 = INFINITY, lo1 = INFINITY, hi0 = -INFINITY, hi1 = -INFINITY;
    for (int i = 0; i < block; ++i) {
      const uint32_t w = src[size_t(i) * (kHeadDim / 2)];
      const float a = bf16_lo(w), c = bf16_hi(w);
      lo0 = fminf(lo0, a);
      hi0 = fmaxf(hi0, a);
      lo1 = fminf(lo1, c);
      hi1 = fmaxf(hi1, c);
    }
    const size_t o = (size_t(rg) * nb + b) * (kHeadDim / 2) + pair;
    bmin[o] = f16_round_down(lo0) | (f16_round_down(lo1) << 16);
    bmax[o] = f16_round_up(hi0) | (f16_round_up(hi1) << 16);
  }
}

}  // namespace sdq

using namespace sdq;

extern "C" int fathom_ingest(const uint16_t* keys, int G, int n, int d, uint32_t* planes,
                             uint32_t* meta, hipStream_t stream) {
  SDQ_REQUIRE(keys && planes && meta, "fathom_ingest: null pointer");
  SDQ_REQUIRE(G >= 1, "fathom_ingest: G=%d must be >= 1", G);
  SDQ_REQUIRE(n >= 64 && n % 64 == 0, "fathom_ingest: n=%d must be a positive multiple of 64", n);
  SDQ_REQUIRE(d == kHeadDim, "fathom_ingest: d=%d unsupported (only 128)", d);
  const int nb64 = n / 64;
  const int bpw = 4;
  dim3 grid(cdiv(nb64, bpw), G);
  hipLaunchKernelGGL(fathom_ingest_kernel, grid, dim3(64), 0, stream,
                     reinterpret_cast<const uint32_t*>(keys), n, nb64, bpw, planes, meta);
  return check_launch("fathom_ingest");
}

extern "C" int minmax_summarize(const uint16_t* keys, int RG, int n, int d, int block,
                                uint16_t* bmin, uint16_t* bmax, hipStream_t stream) {
  SDQ_REQUIRE(keys && bmin && bmax, "minmax_summarize: null pointer");
  SDQ_REQUIRE(RG >= 1, "minmax_summarize: RG=%d must be >= 1", RG);
  SDQ_REQUIRE(block >= 1 && n >= block && n % block == 0,
              "minmax_summarize: n=%d must be a positive multiple of block=%d", n, block);
  SDQ_REQUIRE(d == kHeadDim, "minmax_summarize: d=%d unsupported (only 128)", d);
  const int nb = n / block;
  const int bpw = 8;
  dim3 grid(cdiv(nb, bpw), RG);
  hipLaunchKernelGGL(minmax_summarize_kernel, grid, dim3(64), 0, stream,
                     reinterpret_cast<const uint32_t*>(keys), n, block, nb, bpw,
                     reinterpret_cast<uint32_t*>(bmin), reinterpret_cast<uint32_t*>(bmax));
  return check_launch("minmax_summarize");
}
