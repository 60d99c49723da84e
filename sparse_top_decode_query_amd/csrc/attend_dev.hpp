// Device pieces of the gathered attention (HashAttention study notes, sec.
// 2.1 sparse output formula; sec. 2.5 page-size-one reads): the query
// operand, the row fetch, the online softmax update and the state merge.
//
// A set's rows are cut into 16-row groups.  For each group one wave computes
// the logits of all the query heads sharing the set with four 16x16x32 bf16
// matrix-core products, S^T = K_group * Q'^T over the 128 dims: the 16 rows
// of K are the A operand, bf16 as stored, and Q' holds every head twice, as
// its bf16 rounding and as the bf16 rounding of the remainder, so hi + lo
// carries about 16 significant bits of the float32 query and, with float32
// accumulation, the logits stay close to float32 accuracy.  The output lane
// layout puts head h of rows 4g..4g+3 of the group in lane 16g+h.  The value
// pass is float32 arithmetic on the vector ALUs: lane 16g+c holds dims
// 8c..8c+7 of the same rows 4g..4g+3, so every probability it needs sits in
// its own 16-lane row and arrives by DPP broadcast.  Each lane row keeps an
// online softmax (running max, sum, unnormalised output) in log2 units; the
// four lane rows of a wave and the waves of a workgroup merge by log-sum-exp
// rescaling at the end.
//
// Rows are fetched with bounds-checked buffer loads at 32-bit byte offsets
// into the (request, KV head) slice of K and V; a skipped row gets an offset
// past the slice, which reads zeros without touching memory.
#pragma once
#include "common.hpp"

namespace sdq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kAtGroups = 2;                      // 16-row groups per slab
constexpr int kAtSlab = 16 * kAtGroups;           // rows a wave takes per step
constexpr int kAtMaxTokens = 1 << 23;             // byte offsets in a slice fit 31 bits
constexpr uint32_t kSkipOffset = 0x80000000u;     // past every slice: the load returns 0
constexpr float kNegBig = -3.0e38f;               // running max before any valid row

__host__ __device__ inline size_t attend_partial_floats(int d) { return size_t(d) + 2; }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {   // nearest, ties to even
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// lane 16g + j receives lane 16g + L of its row (L folds to a constant)
__device__ __forceinline__ float row_bcast(float v, int L) {
  switch (L) {
    case 0: return dpp_mov_f32<0x150>(v);
    case 1: return dpp_mov_f32<0x151>(v);
    case 2: return dpp_mov_f32<0x152>(v);
    case 3: return dpp_mov_f32<0x153>(v);
    case 4: return dpp_mov_f32<0x154>(v);
    case 5: return dpp_mov_f32<0x155>(v);
    case 6: return dpp_mov_f32<0x156>(v);
    default: return dpp_mov_f32<0x157>(v);
  }
}

// The K and V slices of one (request, KV head): bounds-checked buffers of n
// rows, so a skipped row's offset reads zeros.
struct AtSlices {
  __amdgpu_buffer_rsrc_t K, V;
};

__device__ __forceinline__ AtSlices at_slices(const uint16_t* K, const uint16_t* V, size_t slice,
                                              int n) {
  AtSlices s;
  s.K = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(K + slice), (short)0, n * 256,
                                          0x00020000);
  s.V = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(V + slice), (short)0, n * 256,
                                          0x00020000);
  return s;
}

// This lane's query values for the B operand Q': column c < NQ is head c,
// column NQ + c the same head again (for its remainder), the others unused
// (zero).  Product kk pairs k-slot 8*g4 + e with dim 8*(4*kk + g4) + e on
// both operands, so a lane reads 16 consecutive bytes of its K row per
// product.  qh0 points at the first query head of the set (16-byte
// aligned): each lane takes its 32 values in eight 16-byte loads, and lanes
// of unused columns load nothing (few load instructions, each touching few
// addresses, at the start of a kernel whose next loads are latency-bound).
template <int NQ>
__device__ __forceinline__ void at_load_q(const float* __restrict__ qh0, float (&qv)[4][8]) {
  const int lane = threadIdx.x & 63, g4 = lane >> 4, col = lane & 15;
  const int hh = col < NQ ? col : (col < 2 * NQ ? col - NQ : -1);
  if (hh >= 0) {
    const float4* qp = reinterpret_cast<const float4*>(qh0 + size_t(hh) * kHeadDim);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float4 a = qp[2 * (4 * kk + g4)], b = qp[2 * (4 * kk + g4) + 1];
      qv[kk][0] = a.x;
      qv[kk][1] = a.y;
      qv[kk][2] = a.z;
      qv[kk][3] = a.w;
      qv[kk][4] = b.x;
      qv[kk][5] = b.y;
      qv[kk][6] = b.z;
      qv[kk][7] = b.w;
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[kk][e] = 0.0f;
  }
}

// Q' from the loaded values: bf16 of the head in columns < NQ, bf16 of the
// remainder in columns NQ..2NQ-1, zeros elsewhere.
template <int NQ>
__device__ __forceinline__ void at_make_qf(const float (&qv)[4][8], bf16x8_t (&qf)[4]) {
  const int col = threadIdx.x & 15;
  const int hh = col < NQ ? col : (col < 2 * NQ ? col - NQ : -1);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u32x4_t w;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t pr[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float x = hh < 0 ? 0.0f : qv[kk][2 * e2 + u];
        const uint32_t hi = f32_to_bf16_bits(x);
        pr[u] = col < NQ ? hi : f32_to_bf16_bits(x - __uint_as_float(hi << 16));
      }
      w[e2] = pr[0] | (pr[1] << 16);
    }
    qf[kk] = __builtin_bit_cast(bf16x8_t, w);
  }
}

// One slab's K and V words: off[0..kAtSlab) are the byte offsets of the
// slab's rows (kSkipOffset: skipped).  K lanes read row 16c + col, value
// lanes rows 16c + 4*g4 + i.  live false: every row skipped (no memory
// access).  vmask bit 4c + i: value row 16c + 4*g4 + i is a real row.
__device__ __forceinline__ void at_fetch(const AtSlices& sl, const uint32_t* off, bool live,
                                         u32x4_t (&kw)[kAtGroups][4], u32x4_t (&vw)[kAtGroups][4],
                                         uint32_t& vmask) {
  const int lane = threadIdx.x & 63, g4 = lane >> 4, col = lane & 15;
  vmask = 0;
#pragma unroll
  for (int c = 0; c < kAtGroups; ++c) {
    const uint32_t ko_l = off[16 * c + col];                   // unconditional read
    const uint32_t ko = live ? ko_l : kSkipOffset;
    const u32x4_t vo4 = *reinterpret_cast<const u32x4_t*>(&off[16 * c + 4 * g4]);
    const uint32_t kb = ko == kSkipOffset ? kSkipOffset : ko + 16u * g4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      kw[c][kk] = __builtin_bit_cast(u32x4_t,
                                     __builtin_amdgcn_raw_buffer_load_b128(sl.K, kb + 64u * kk, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t vo = live ? vo4[i] : kSkipOffset;
      vmask |= uint32_t(vo != kSkipOffset) << (4 * c + i);
      const uint32_t vb = vo == kSkipOffset ? kSkipOffset : vo + 16u * col;
      vw[c][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sl.V, vb, 0, 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);        // keep the loads ahead of the work that follows
}

// A lane row's online softmax state: lane 16*g4 + h holds m and l of head h;
// o[h][e] is dim 8*col + e of head h.
template <int NQ>
struct AtState {
  float m, l;
  float o[NQ][8];
};

template <int NQ>
__device__ __forceinline__ void at_init(AtState<NQ>& s) {
  s.m = kNegBig;
  s.l = 0.0f;
#pragma unroll
  for (int h = 0; h < NQ; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) s.o[h][e] = 0.0f;
}

// Adds one slab to the state: rows whose bit 4c + i of cmask is clear (value
// rows 16c + 4*g4 + i) take no part.
template <int NQ>
__device__ __forceinline__ void at_compute(AtState<NQ>& s, const bf16x8_t (&qf)[4],
                                           const u32x4_t (&kc)[kAtGroups][4],
                                           const u32x4_t (&vc)[kAtGroups][4], uint32_t cmask,
                                           float scale_log2) {
  // logits: lane 16*g4 + h gets head h of rows 4*g4 + i of group c
  float x[kAtGroups][4];
#pragma unroll
  for (int c = 0; c < kAtGroups; ++c) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kc[c][kk]),
                                                    qf[kk], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = acc[i] + dpp_mov_f32<0x100 + NQ>(acc[i]);   // hi column + lo column
      x[c][i] = ((cmask >> (4 * c + i)) & 1u) ? z * scale_log2 : -INFINITY;
    }
  }
  float cm = x[0][0];
#pragma unroll
  for (int c = 0; c < kAtGroups; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) cm = fmaxf(cm, x[c][i]);
  const float mn = fmaxf(s.m, cm);
  const float alpha = __builtin_amdgcn_exp2f(s.m - mn);     // 1 while no row was valid
  float p[kAtGroups][4];
  float ps = 0.0f;
#pragma unroll
  for (int c = 0; c < kAtGroups; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[c][i] = __builtin_amdgcn_exp2f(x[c][i] - mn);     // 0 for skipped rows
      ps += p[c][i];
    }
  s.l = __builtin_fmaf(s.l, alpha, ps);
  s.m = mn;
  // values: lane 16*g4 + col, dims 8*col .. 8*col+7 of the same rows
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    const float ah = row_bcast(alpha, h);
#pragma unroll
    for (int e = 0; e < 8; ++e) s.o[h][e] *= ah;
  }
#pragma unroll
  for (int c = 0; c < kAtGroups; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t w = vc[c][i];
      const float vf[8] = {bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1]),
                           bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
#pragma unroll
      for (int h = 0; h < NQ; ++h) {
        const float ph = row_bcast(p[c][i], h);
#pragma unroll
        for (int e = 0; e < 8; ++e) s.o[h][e] = __builtin_fmaf(ph, vf[e], s.o[h][e]);
      }
    }
}

// Lane row `sr`'s state into st[sr][NQ][d + 2] (o, then m and l).
template <int NQ>
__device__ __forceinline__ void at_store_state(const AtState<NQ>& s, float* st, int sr) {
  const int col = threadIdx.x & 15;
#pragma unroll
  for (int h = 0; h < NQ; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) st[(sr * NQ + h) * (kHeadDim + 2) + 8 * col + e] = s.o[h][e];
  if (col < NQ) {
    st[(sr * NQ + col) * (kHeadDim + 2) + kHeadDim] = s.m;
    st[(sr * NQ + col) * (kHeadDim + 2) + kHeadDim + 1] = s.l;
  }
}

// Merges the nst lane-row states of head h, dim dd: returns the unnormalised
// output, with the merged maximum (log2 units) and sum in Mx and L.
template <int NQ, int NST>
__device__ __forceinline__ float at_merge_states(const float* st, int h, int dd, float& Mx,
                                                 float& L) {
  Mx = kNegBig;
#pragma unroll
  for (int w = 0; w < NST; ++w) Mx = fmaxf(Mx, st[(w * NQ + h) * (kHeadDim + 2) + kHeadDim]);
  L = 0.0f;
  float acc = 0.0f;
#pragma unroll
  for (int w = 0; w < NST; ++w) {
    const float* sw = st + (w * NQ + h) * (kHeadDim + 2);
    const float f = __builtin_amdgcn_exp2f(sw[kHeadDim] - Mx);
    L = __builtin_fmaf(sw[kHeadDim + 1], f, L);
    acc = __builtin_fmaf(sw[dd], f, acc);
  }
  return acc;
}

}  // namespace sdq
