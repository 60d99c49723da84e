// Index construction from the bf16 key cache:
//  * fathom_ingest: per-channel 4-bit block quantiser and channel-major bit
//    planes (Fathom summary, bit-plane paragraph);
//  * minmax_summarize: per-block min/max key summaries (OasisKV review,
//    Quest-style block summaries).
// Both build a whole index before decoding; fathom_append and minmax_append
// add a decode step's new tokens to a cache of fixed row capacity, quantising
// (or summarising) the open block again until it is full.  None of them is
// part of the timed decode path.
#include "common.hpp"

namespace sdq {

// One workgroup of 1024 threads per (KV head, 64-token block).  The block's
// 64 key rows (16 KB) come in as one coalesced 16-byte load per thread and are
// staged in LDS.  Thread (j, q) takes channel j and the eight tokens
// 8q..8q+7: their min and max go to LDS, every thread then reduces the eight
// partials of its channel, codes its eight tokens (one IEEE division each)
// and ORs their bits into the block's plane words in LDS; 128 threads write
// the 2 words x 4 planes of each channel and its metadata.  A workgroup
// covers blocks [b0, b0 + nblk) of one head along gridDim.x.
//
// Rows are n_cap tokens long (the cache's capacity) and the first n tokens
// are present.  A partly filled last block (the open block of a growing
// cache) is quantised over its m present tokens: rows past them are staged as
// copies of the last present row, which leaves the block's min and max
// unchanged, and the absent tokens' plane bits are cleared.
constexpr int kApThreads = 1024;

__global__ __launch_bounds__(kApThreads) void fathom_append_kernel(
    const uint4* __restrict__ keys, int n_cap, int n, int b0, uint32_t* __restrict__ planes,
    uint32_t* __restrict__ meta) {
  __shared__ uint16_t s_k[64][kHeadDim];
  __shared__ float s_mn[8][kHeadDim], s_mx[8][kHeadDim];
  __shared__ uint32_t s_w[kHeadDim][8];                   // [channel][plane * 2 + half]
  const int g = blockIdx.y;
  const int b = b0 + blockIdx.x;
  const int t = threadIdx.x;
  const int m = n - b * 64 < 64 ? n - b * 64 : 64;          // present tokens, >= 1
  const uint4* src = keys + (size_t(g) * n_cap + size_t(b) * 64) * (kHeadDim / 8);
  {
    const int row = t >> 4;                                  // 16 pieces of 16 bytes per row
    const uint4 v = src[size_t(row < m ? row : m - 1) * (kHeadDim / 8) + (t & 15)];
    reinterpret_cast<uint4*>(&s_k[row][0])[t & 15] = v;
  }
  const int j = t & (kHeadDim - 1);
  const int qd = t >> 7;                                     // tokens 8qd..8qd+7
  (&s_w[0][0])[t] = 0u;                                      // 1024 words, one per thread
  __syncthreads();
  float x[8];
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = __uint_as_float(uint32_t(s_k[8 * qd + i][j]) << 16);
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  s_mn[qd][j] = mn;
  s_mx[qd][j] = mx;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    mn = fminf(mn, s_mn[u][j]);
    mx = fmaxf(mx, s_mx[u][j]);
  }
  const _Float16 off16 = _Float16(mn);
  const _Float16 sc16 = _Float16(__fdiv_rn(mx - mn, 15.0f));
  const float off = float(off16);
  const float sc = float(sc16);
  uint32_t bits[4] = {0, 0, 0, 0};                           // this thread's 8 tokens, per plane
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float r = (sc == 0.0f) ? 0.0f : rintf(__fdiv_rn(x[i] - off, sc));
    r = fminf(fmaxf(r, 0.0f), 15.0f);
    const uint32_t code = 8 * qd + i < m ? uint32_t(r) : 0u; // absent tokens hold code 0
#pragma unroll
    for (int p = 0; p < 4; ++p) bits[p] |= ((code >> (3 - p)) & 1u) << i;
  }
  const int half = qd >> 2, sh = 8 * (qd & 3);               // position inside the 32-token word
#pragma unroll
  for (int p = 0; p < 4; ++p) atomicOr(&s_w[j][p * 2 + half], bits[p] << sh);
  __syncthreads();
  if (t < kHeadDim) {
    const size_t nw = size_t(n_cap) / 32;                    // 32-token words per plane row
    uint32_t* prow = planes + (size_t(g) * kHeadDim + t) * 4 * nw + 2 * size_t(b);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      prow[size_t(p) * nw] = s_w[t][p * 2];
      prow[size_t(p) * nw + 1] = s_w[t][p * 2 + 1];
    }
    meta[(size_t(g) * kHeadDim + t) * (n_cap / 64) + b] =
        uint32_t(__builtin_bit_cast(uint16_t, sc16)) |
        (uint32_t(__builtin_bit_cast(uint16_t, off16)) << 16);
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

// One thread per adjacent channel pair; a workgroup walks `bpw` blocks of the
// range [b0, b0 + nblk).  Rows are n_cap tokens long with the first n
// present; a partly filled last block is summarised over its present tokens.
__global__ __launch_bounds__(64) void minmax_append_kernel(const uint32_t* __restrict__ keys,
                                                           int n_cap, int n, int block, int b0,
                                                           int nblk, int bpw,
                                                           uint32_t* __restrict__ bmin,
                                                           uint32_t* __restrict__ bmax) {
  const int rg = blockIdx.y;
  const int pair = threadIdx.x;
  const int nb_cap = n_cap / block;
  for (int bb = 0; bb < bpw; ++bb) {
    const int bi = blockIdx.x * bpw + bb;
    if (bi >= nblk) break;
    const int b = b0 + bi;
    const int m = n - b * block < block ? n - b * block : block;
    const uint32_t* src = keys + (size_t(rg) * n_cap + size_t(b) * block) * (kHeadDim / 2) + pair;
    float lo0 = INFINITY, lo1 = INFINITY, hi0 = -INFINITY, hi1 = -INFINITY;
    // rows in batches of 16, every load of a batch issued before the first
    // use; rows past m repeat row m - 1, which leaves min and max unchanged
    for (int i0 = 0; i0 < m; i0 += 16) {
      uint32_t w[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        w[u] = src[size_t(i0 + u < m ? i0 + u : m - 1) * (kHeadDim / 2)];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float a = bf16_lo(w[u]), c = bf16_hi(w[u]);
        lo0 = fminf(lo0, a);
        hi0 = fmaxf(hi0, a);
        lo1 = fminf(lo1, c);
        hi1 = fmaxf(hi1, c);
      }
    }
    const size_t o = (size_t(rg) * nb_cap + b) * (kHeadDim / 2) + pair;
    bmin[o] = f16_round_down(lo0) | (f16_round_down(lo1) << 16);
    bmax[o] = f16_round_up(hi0) | (f16_round_up(hi1) << 16);
  }
}

}  // namespace sdq

using namespace sdq;

static void launch_fathom_append(const uint16_t* keys, int G, int n_cap, int n, int b0, int nblk,
                                 uint32_t* planes, uint32_t* meta, hipStream_t stream) {
  dim3 grid(nblk, G);
  hipLaunchKernelGGL(fathom_append_kernel, grid, dim3(kApThreads), 0, stream,
                     reinterpret_cast<const uint4*>(keys), n_cap, n, b0, planes, meta);
}

extern "C" int fathom_ingest(const uint16_t* keys, int G, int n, int d, uint32_t* planes,
                             uint32_t* meta, hipStream_t stream) {
  SDQ_REQUIRE(keys && planes && meta, "fathom_ingest: null pointer");
  SDQ_REQUIRE(G >= 1, "fathom_ingest: G=%d must be >= 1", G);
  SDQ_REQUIRE(n >= 64 && n % 64 == 0, "fathom_ingest: n=%d must be a positive multiple of 64", n);
  SDQ_REQUIRE(n < (1 << 25), "fathom_ingest: n=%d must be below 2^25", n);
  SDQ_REQUIRE(d == kHeadDim, "fathom_ingest: d=%d unsupported (only 128)", d);
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(keys) % 16 == 0, "fathom_ingest: keys must be 16-byte aligned");
  launch_fathom_append(keys, G, n, n, 0, n / 64, planes, meta, stream);
  return check_launch("fathom_ingest");
}

extern "C" int fathom_append(const uint16_t* keys, int G, int d, int n_cap, int n_old, int n_new,
                             uint32_t* planes, uint32_t* meta, hipStream_t stream) {
  SDQ_REQUIRE(keys && planes && meta, "fathom_append: null pointer");
  SDQ_REQUIRE(G >= 1, "fathom_append: G=%d must be >= 1", G);
  SDQ_REQUIRE(d == kHeadDim, "fathom_append: d=%d unsupported (only 128)", d);
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(keys) % 16 == 0, "fathom_append: keys must be 16-byte aligned");
  SDQ_REQUIRE(n_cap >= 64 && n_cap % 64 == 0 && n_cap < (1 << 25),
              "fathom_append: n_cap=%d must be a positive multiple of 64 below 2^25", n_cap);
  SDQ_REQUIRE(n_old >= 0 && n_new >= 0 && (long long)n_old + n_new <= n_cap,
              "fathom_append: n_old=%d + n_new=%d must fit n_cap=%d", n_old, n_new, n_cap);
  if (n_new == 0) return SDQ_OK;
  const int n = n_old + n_new;
  const int b0 = n_old / 64;
  launch_fathom_append(keys, G, n_cap, n, b0, (n + 63) / 64 - b0, planes, meta, stream);
  return check_launch("fathom_append");
}

static void launch_minmax_append(const uint16_t* keys, int RG, int n_cap, int n, int block, int b0,
                                 int nblk, uint16_t* bmin, uint16_t* bmax, hipStream_t stream) {
  const int bpw = 8;
  dim3 grid(cdiv(nblk, bpw), RG);
  hipLaunchKernelGGL(minmax_append_kernel, grid, dim3(64), 0, stream,
                     reinterpret_cast<const uint32_t*>(keys), n_cap, n, block, b0, nblk, bpw,
                     reinterpret_cast<uint32_t*>(bmin), reinterpret_cast<uint32_t*>(bmax));
}

extern "C" int minmax_summarize(const uint16_t* keys, int RG, int n, int d, int block,
                                uint16_t* bmin, uint16_t* bmax, hipStream_t stream) {
  SDQ_REQUIRE(keys && bmin && bmax, "minmax_summarize: null pointer");
  SDQ_REQUIRE(RG >= 1, "minmax_summarize: RG=%d must be >= 1", RG);
  SDQ_REQUIRE(block >= 1 && n >= block && n % block == 0,
              "minmax_summarize: n=%d must be a positive multiple of block=%d", n, block);
  SDQ_REQUIRE(d == kHeadDim, "minmax_summarize: d=%d unsupported (only 128)", d);
  launch_minmax_append(keys, RG, n, n, block, 0, n / block, bmin, bmax, stream);
  return check_launch("minmax_summarize");
}

extern "C" int minmax_append(const uint16_t* keys, int RG, int d, int n_cap, int n_old, int n_new,
                             int block, uint16_t* bmin, uint16_t* bmax, hipStream_t stream) {
  SDQ_REQUIRE(keys && bmin && bmax, "minmax_append: null pointer");
  SDQ_REQUIRE(RG >= 1, "minmax_append: RG=%d must be >= 1", RG);
  SDQ_REQUIRE(d == kHeadDim, "minmax_append: d=%d unsupported (only 128)", d);
  SDQ_REQUIRE(block >= 1 && n_cap >= block && n_cap % block == 0,
              "minmax_append: n_cap=%d must be a positive multiple of block=%d", n_cap, block);
  SDQ_REQUIRE(n_old >= 0 && n_new >= 0 && (long long)n_old + n_new <= n_cap,
              "minmax_append: n_old=%d + n_new=%d must fit n_cap=%d", n_old, n_new, n_cap);
  if (n_new == 0) return SDQ_OK;
  const int n = n_old + n_new;
  const int b0 = n_old / block;
  launch_minmax_append(keys, RG, n_cap, n, block, b0, (n + block - 1) / block - b0, bmin, bmax,
                       stream);
  return check_launch("minmax_append");
}
