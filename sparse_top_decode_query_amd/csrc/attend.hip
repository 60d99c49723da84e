// Renormalised softmax attention over rows read by index (HashAttention
// study notes, sec. 2.1 sparse output formula; sec. 2.5 page-size-one reads:
// the selected rows are read in place by index, a 256-byte bf16 row being
// more than a cache line).
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
// four lane rows of a wave, the waves of a workgroup and, for sets split over
// several workgroups, the splits merge by log-sum-exp rescaling at the end.
//
// Rows are fetched with bounds-checked buffer loads at 32-bit byte offsets
// into the (request, KV head) slice of K and V; a skipped row gets an offset
// past the slice, which reads zeros without touching memory.  Each wave
// requests its next 32 rows before it works on the current 32.
#include "common.hpp"

namespace sdq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kAtWaves = 4;
constexpr int kAtThreads = 64 * kAtWaves;
constexpr int kAtGroups = 2;                      // 16-row groups per slab
constexpr int kAtSlab = 16 * kAtGroups;           // rows a wave takes per step
constexpr int kAtMaxTokens = 1 << 23;             // byte offsets in a slice fit 31 bits
constexpr uint32_t kSkipOffset = 0x80000000u;     // past every slice: the load returns 0
constexpr float kNegBig = -3.0e38f;               // running max before any valid row
constexpr int kAtMaxRows = 4096;                  // rows per workgroup (offsets kept in LDS)
constexpr int kAtFill = 8;                        // row offsets per thread per fill pass

struct AttendArgs {
  const float* q;
  const uint16_t* K;
  const uint16_t* V;
  const int32_t* idx;
  int R, Hq, Hkv, per_qh, n, n_cap, n_idx, bt, bt_shift, nblk, rows_per_split;
  float scale_log2;     // softmax scale * log2(e)
  float* parts;         // partials [R*Hq][nsplit][d + 2] when a set is split (workspace)
  float* out;
};

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

// Merges the nsplit partials of one query head (dim dd) in one pass with a
// running maximum, kCb partials at a time with each batch's loads issued
// together (one memory round trip per batch).
__device__ float merge_splits(const float* __restrict__ base, int nsplit, int dd) {
  constexpr int kCb = 16;
  const size_t pf = attend_partial_floats(kHeadDim);
  float M = kNegBig, L = 0.0f, acc = 0.0f;
  for (int c0 = 0; c0 < nsplit; c0 += kCb) {
    float mv[kCb], lv[kCb], ov[kCb];
#pragma unroll
    for (int e = 0; e < kCb; ++e) {
      const float* pc = base + size_t(c0 + e < nsplit ? c0 + e : 0) * pf;
      mv[e] = pc[kHeadDim];
      lv[e] = pc[kHeadDim + 1];
      ov[e] = pc[dd];
    }
    float Mb = M;
#pragma unroll
    for (int e = 0; e < kCb; ++e) Mb = c0 + e < nsplit ? fmaxf(Mb, mv[e]) : Mb;
    const float r = __builtin_amdgcn_exp2f(M - Mb);          // rescale what came before
    L *= r;
    acc *= r;
#pragma unroll
    for (int e = 0; e < kCb; ++e) {
      const float w = c0 + e < nsplit ? __builtin_amdgcn_exp2f(mv[e] - Mb) : 0.0f;
      L = __builtin_fmaf(lv[e], w, L);
      acc = __builtin_fmaf(ov[e], w, acc);
    }
    M = Mb;
  }
  return (L > 0.0f) ? acc / L : 0.0f;
}

// One workgroup per query head of a split call: merges its partials.
__global__ __launch_bounds__(kHeadDim) void attend_combine_kernel(const float* __restrict__ parts,
                                                                  int nsplit,
                                                                  float* __restrict__ out) {
  const int qh = blockIdx.x, dd = threadIdx.x;
  out[size_t(qh) * kHeadDim + dd] =
      merge_splits(parts + size_t(qh) * nsplit * attend_partial_floats(kHeadDim), nsplit, dd);
}

template <int NQ, bool POW2>
__global__ __launch_bounds__(kAtThreads) void attend_kernel(AttendArgs a) {
  constexpr int W = kAtWaves;
  // row byte offsets while the rows are read, then the lane-row states
  constexpr int kStates = W * 4;
  constexpr int kStateFloats = kStates * NQ * (kHeadDim + 2);
  __shared__ __attribute__((aligned(16))) uint32_t s_lds[kAtMaxRows > kStateFloats ? kAtMaxRows : kStateFloats];
  uint32_t* s_off = s_lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar control flow
  const int g4 = lane >> 4;                 // lane row: rows 4*g4 .. 4*g4+3 of a group
  const int col = lane & 15;                // MFMA column; value dims 8*col .. 8*col+7
  const int split = blockIdx.x, set = blockIdx.y;
  const int nsplit = gridDim.x;
  const int Hsel = a.per_qh ? a.Hq : a.Hkv;
  const int r = set / Hsel, hs = set % Hsel;
  const int grp = a.Hq / a.Hkv;
  const int kvh = a.per_qh ? hs / grp : hs;
  const int h0 = a.per_qh ? hs : hs * grp;  // first query head of the set
  const int M = a.n_idx * a.bt;
  const int rb = split * a.rows_per_split;
  const int re = min(M, rb + a.rows_per_split);
  const int nslab = (re - rb + kAtSlab - 1) / kAtSlab;
  const int32_t* sidx = a.idx + size_t(set) * a.n_idx;
  const size_t slice = (size_t(r) * a.Hkv + kvh) * size_t(a.n_cap) * kHeadDim;
  const __amdgpu_buffer_rsrc_t Kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.K + slice), (short)0, a.n * 256, 0x00020000);
  const __amdgpu_buffer_rsrc_t Vr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.V + slice), (short)0, a.n * 256, 0x00020000);

  // Q' as the B operand: column c < NQ is head c rounded to bf16, column
  // NQ + c the rounded remainder, the others zero.  Product kk pairs k-slot
  // 8*g4 + e with dim 8*(4*kk + g4) + e on both operands, so a lane reads 16
  // consecutive bytes of its K row per product.  The query loads go out
  // first, together with the idx loads of the row offsets below.
  const int hh = col < NQ ? col : (col < 2 * NQ ? col - NQ : -1);
  float qv[4][8];
  {
    const float* qp = a.q + (size_t(r) * a.Hq + h0 + (hh < 0 ? 0 : hh)) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[kk][e] = qp[8 * (4 * kk + g4) + e];
  }
  __builtin_amdgcn_sched_barrier(0);

  // byte offset of every row of this workgroup, computed once from idx
  for (int i0 = 0; i0 < nslab * kAtSlab; i0 += kAtThreads * kAtFill) {
    int ent[kAtFill];
#pragma unroll
    for (int u = 0; u < kAtFill; ++u) {       // all of a pass's idx loads first
      const int row = rb + i0 + u * kAtThreads + tid;
      const int rr = row < re ? row : re - 1;
      ent[u] = sidx[POW2 ? (rr >> a.bt_shift) : rr / a.bt];
    }
#pragma unroll
    for (int u = 0; u < kAtFill; ++u) {
      const int li = i0 + u * kAtThreads + tid;
      if (li < nslab * kAtSlab) {
        const int row = rb + li;
        const int rr = row < re ? row : re - 1;
        const int blk = POW2 ? (rr >> a.bt_shift) : rr / a.bt;
        const bool ok = row < re && unsigned(ent[u]) < unsigned(a.nblk);
        const uint32_t t = uint32_t(ok ? ent[u] : 0) * uint32_t(a.bt) + uint32_t(rr - blk * a.bt);
        s_off[li] = ok && t < uint32_t(a.n) ? t << 8 : kSkipOffset;
      }
    }
  }

  bf16x8_t qf[4];
  {
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
  __syncthreads();

  // slab s of this wave: local rows (wave + s * W) * kAtSlab + 16c + ...
  //   K lanes: row 16c + col;  value lanes: rows 16c + 4*g4 + i
  const int my_slabs = wave < nslab ? (nslab - wave + W - 1) / W : 0;
  auto fetch = [&](int s, u32x4_t (&kw)[kAtGroups][4], u32x4_t (&vw)[kAtGroups][4],
                   uint32_t& vmask) {
    const bool live = s < my_slabs;           // past the wave's last slab: skipped rows
    const int base = (wave + (live ? s : 0) * W) * kAtSlab;
    vmask = 0;
#pragma unroll
    for (int c = 0; c < kAtGroups; ++c) {
      const uint32_t ko_l = s_off[base + 16 * c + col];        // unconditional read
      const uint32_t ko = live ? ko_l : kSkipOffset;
      const u32x4_t vo4 = *reinterpret_cast<const u32x4_t*>(&s_off[base + 16 * c + 4 * g4]);
      const uint32_t kb = ko == kSkipOffset ? kSkipOffset : ko + 16u * g4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kw[c][kk] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(Kr, kb + 64u * kk, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t vo = live ? vo4[i] : kSkipOffset;
        vmask |= uint32_t(vo != kSkipOffset) << (4 * c + i);
        const uint32_t vb = vo == kSkipOffset ? kSkipOffset : vo + 16u * col;
        vw[c][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(Vr, vb, 0, 0));
      }
    }
    __builtin_amdgcn_sched_barrier(0);        // keep the loads ahead of the work that follows
  };

  float m = kNegBig, l = 0.0f;              // lane 16*g4 + h: head h of the lane row
  float o[NQ][8];
#pragma unroll
  for (int h = 0; h < NQ; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;

  auto compute = [&](const u32x4_t (&kc)[kAtGroups][4], const u32x4_t (&vc)[kAtGroups][4],
                     uint32_t cmask) {
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
        x[c][i] = ((cmask >> (4 * c + i)) & 1u) ? z * a.scale_log2 : -INFINITY;
      }
    }
    float cm = x[0][0];
#pragma unroll
    for (int c = 0; c < kAtGroups; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) cm = fmaxf(cm, x[c][i]);
    const float mn = fmaxf(m, cm);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);     // 1 while no row was valid
    float p[kAtGroups][4];
    float ps = 0.0f;
#pragma unroll
    for (int c = 0; c < kAtGroups; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[c][i] = __builtin_amdgcn_exp2f(x[c][i] - mn);     // 0 for skipped rows
        ps += p[c][i];
      }
    l = __builtin_fmaf(l, alpha, ps);
    m = mn;
    // values: lane 16*g4 + col, dims 8*col .. 8*col+7 of the same rows
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      const float ah = row_bcast(alpha, h);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= ah;
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
          for (int e = 0; e < 8; ++e) o[h][e] = __builtin_fmaf(ph, vf[e], o[h][e]);
        }
      }
  };

  // two register buffers: the next slab is requested before the current one
  // is used (slabs past the wave's last read as skipped rows: no memory access)
  if (my_slabs > 0) {
    u32x4_t kA[kAtGroups][4], vA[kAtGroups][4], kB[kAtGroups][4], vB[kAtGroups][4];
    uint32_t mA, mB;
    fetch(0, kA, vA, mA);
    for (int s = 0; s < my_slabs; s += 2) {
      fetch(s + 1, kB, vB, mB);
      compute(kA, vA, mA);
      fetch(s + 2, kA, vA, mA);
      if (s + 1 < my_slabs) compute(kB, vB, mB);
    }
  }

  // every lane row's state (m and l of head h in its lane 16*g4 + h, o spread
  // over its 16 lanes) goes to LDS once all waves are done with the offsets
  __syncthreads();
  float* st = reinterpret_cast<float*>(s_lds);               // [kStates][NQ][d + 2]
  const int sr = wave * 4 + g4;
#pragma unroll
  for (int h = 0; h < NQ; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) st[(sr * NQ + h) * (kHeadDim + 2) + 8 * col + e] = o[h][e];
  if (col < NQ) {
    st[(sr * NQ + col) * (kHeadDim + 2) + kHeadDim] = m;
    st[(sr * NQ + col) * (kHeadDim + 2) + kHeadDim + 1] = l;
  }
  __syncthreads();
  // merge the states: one thread per (head, dim); write the output, or the
  // split's partial (unnormalised output, max in log2 units, sum)
  const size_t pf = attend_partial_floats(kHeadDim);
  float* parts = a.parts;
  for (int xi = tid; xi < NQ * kHeadDim; xi += kAtThreads) {
    const int h = xi / kHeadDim, dd = xi % kHeadDim;
    float Mx = kNegBig;
#pragma unroll
    for (int w = 0; w < kStates; ++w) Mx = fmaxf(Mx, st[(w * NQ + h) * (kHeadDim + 2) + kHeadDim]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kStates; ++w) {
      const float* sw = st + (w * NQ + h) * (kHeadDim + 2);
      const float f = __builtin_amdgcn_exp2f(sw[kHeadDim] - Mx);
      L = __builtin_fmaf(sw[kHeadDim + 1], f, L);
      acc = __builtin_fmaf(sw[dd], f, acc);
    }
    const size_t qh = size_t(r) * a.Hq + h0 + h;
    if (nsplit == 1) {
      a.out[qh * kHeadDim + dd] = (L > 0.0f) ? acc / L : 0.0f;
    } else {
      float* dst = parts + (qh * nsplit + split) * pf;
      dst[dd] = acc;
      if (dd == 0) {
        dst[kHeadDim] = Mx;
        dst[kHeadDim + 1] = L;
      }
    }
  }
}

}  // namespace sdq

using namespace sdq;

// Rows per workgroup.  A wave's slabs are fetched one ahead, so a long set
// in one workgroup costs about one memory round trip per slab per wave: few
// sets are split over about kAtTargetWgs workgroups of whole 128-row units
// (a slab per wave at least) and merged by the combine kernel, which costs
// less.  Enough sets to fill the chip take one workgroup each (no combine).
// No workgroup takes more than kAtMaxRows rows.
constexpr int kAtTargetWgs = 512;

static long long attend_rows_per_split(long long sets, long long M) {
  const long long unit = (long long)kAtWaves * kAtSlab;
  long long per = M;
  if (sets < kAtTargetWgs / 2) {
    per = (sets * M + kAtTargetWgs - 1) / kAtTargetWgs;
    per = (per + unit - 1) / unit * unit;
  }
  if (per > kAtMaxRows) per = kAtMaxRows;
  return per < M ? per : M;
}

static long long attend_nsplit(long long sets, long long M) {
  const long long per = attend_rows_per_split(sets, M);
  return (M + per - 1) / per;
}

extern "C" size_t gather_attend_workspace_bytes(int R, int H_q, int H_kv, int sets_per_query_head,
                                                int n_idx, int block_tokens, int d) {
  if (R < 1 || H_q < 1 || H_kv < 1 || n_idx < 1 || block_tokens < 1 || d != kHeadDim) return 0;
  const long long sets = (long long)R * (sets_per_query_head ? H_q : H_kv);
  const long long nsplit = attend_nsplit(sets, (long long)n_idx * block_tokens);
  if (nsplit <= 1) return 0;
  return size_t(R) * H_q * size_t(nsplit) * attend_partial_floats(d) * sizeof(float);
}

template <int NQ>
static void launch_attend(dim3 grid, bool pow2, const AttendArgs& a, hipStream_t stream) {
  if (pow2)
    hipLaunchKernelGGL((attend_kernel<NQ, true>), grid, dim3(kAtThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attend_kernel<NQ, false>), grid, dim3(kAtThreads), 0, stream, a);
}

static int attend_impl(const char* nm, const float* q, const uint16_t* K, const uint16_t* V,
                       const int32_t* idx, int R, int H_q, int H_kv, int sets_per_query_head,
                       int n, int n_cap, int n_idx, int block_tokens, int d, float softmax_scale,
                       float* out, void* ws, size_t ws_bytes, hipStream_t stream);

extern "C" int gather_attend(const float* q, const uint16_t* K, const uint16_t* V,
                             const int32_t* idx, int R, int H_q, int H_kv, int sets_per_query_head,
                             int n, int n_cap, int n_idx, int block_tokens, int d,
                             float softmax_scale, float* out, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  return attend_impl("gather_attend", q, K, V, idx, R, H_q, H_kv, sets_per_query_head, n, n_cap,
                     n_idx, block_tokens, d, softmax_scale, out, ws, ws_bytes, stream);
}

// K and V stay in pinned host memory: the same kernel reads the selected rows
// through the buffers' device mapping, over the host link.
extern "C" int gather_attend_host_kv(const float* q, const uint16_t* K_host,
                                     const uint16_t* V_host, const int32_t* idx, int R, int H_q,
                                     int H_kv, int sets_per_query_head, int n, int n_cap,
                                     int n_idx, int block_tokens, int d, float softmax_scale,
                                     float* out,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  SDQ_REQUIRE(K_host && V_host, "gather_attend_host_kv: null pointer");
  void* kd = nullptr;
  void* vd = nullptr;
  if (hipHostGetDevicePointer(&kd, const_cast<uint16_t*>(K_host), 0) != hipSuccess || !kd ||
      hipHostGetDevicePointer(&vd, const_cast<uint16_t*>(V_host), 0) != hipSuccess || !vd) {
    (void)hipGetLastError();
    set_error("gather_attend_host_kv: K and V must be pinned, device-mapped host memory");
    return SDQ_EINVAL;
  }
  return attend_impl("gather_attend_host_kv", q, static_cast<const uint16_t*>(kd),
                     static_cast<const uint16_t*>(vd), idx, R, H_q, H_kv, sets_per_query_head, n,
                     n_cap, n_idx, block_tokens, d, softmax_scale, out, ws, ws_bytes, stream);
}

static int attend_impl(const char* nm, const float* q, const uint16_t* K, const uint16_t* V,
                       const int32_t* idx, int R, int H_q, int H_kv, int sets_per_query_head,
                       int n, int n_cap, int n_idx, int block_tokens, int d, float softmax_scale,
                       float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  SDQ_REQUIRE(q && K && V && idx && out, "%s: null pointer", nm);
  SDQ_REQUIRE(n <= n_cap, "%s: n=%d exceeds the row capacity n_cap=%d", nm, n, n_cap);
  SDQ_REQUIRE(R >= 1 && H_q >= 1 && H_kv >= 1 && n >= 1 && n_idx >= 1 && block_tokens >= 1,
              "%s: R, H_q, H_kv, n, n_idx, block_tokens must be >= 1", nm);
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(K) % 16 == 0 && reinterpret_cast<uintptr_t>(V) % 16 == 0,
              "%s: K and V must be 16-byte aligned", nm);
  SDQ_REQUIRE(H_q % H_kv == 0, "%s: H_q=%d not a multiple of H_kv=%d", nm, H_q, H_kv);
  SDQ_REQUIRE(d == kHeadDim, "%s: d=%d unsupported (only 128)", nm, d);
  SDQ_REQUIRE(n < kAtMaxTokens, "%s: n=%d tokens per head exceeds %d", nm, n,
              kAtMaxTokens - 1);
  SDQ_REQUIRE((long long)n_idx * block_tokens <= 0x7FFFFFFFLL, "%s: too many rows", nm);
  const int grp = H_q / H_kv;
  const int NQ = sets_per_query_head ? 1 : grp;
  SDQ_REQUIRE(NQ == 1 || NQ == 2 || NQ == 4 || NQ == 8,
              "%s: %d query heads per set unsupported (1, 2, 4 or 8)", nm, NQ);
  const long long sets = (long long)R * (sets_per_query_head ? H_q : H_kv);
  SDQ_REQUIRE(sets <= 65535, "%s: %lld index sets exceed 65535", nm, sets);
  const size_t need = gather_attend_workspace_bytes(R, H_q, H_kv, sets_per_query_head, n_idx,
                                                    block_tokens, d);
  SDQ_REQUIRE(need == 0 || (ws && ws_bytes >= need),
              "%s: workspace of %zu bytes needed, %zu given", nm, need, ws_bytes);
  const long long M = (long long)n_idx * block_tokens;
  const long long per = attend_rows_per_split(sets, M);
  const long long nsplit = (M + per - 1) / per;
  const bool pow2 = (block_tokens & (block_tokens - 1)) == 0;
  int shift = 0;
  while ((1 << shift) < block_tokens && shift < 30) ++shift;
  const int nblk = int((n + (long long)block_tokens - 1) / block_tokens);
  AttendArgs a{q, K, V, idx, R, H_q, H_kv, sets_per_query_head ? 1 : 0, n, n_cap, n_idx, block_tokens,
               shift, nblk, int(per), softmax_scale * 1.4426950408889634f,
               reinterpret_cast<float*>(ws), out};
  const dim3 grid{unsigned(nsplit), unsigned(sets), 1u};
  switch (NQ) {
    case 1: launch_attend<1>(grid, pow2, a, stream); break;
    case 2: launch_attend<2>(grid, pow2, a, stream); break;
    case 4: launch_attend<4>(grid, pow2, a, stream); break;
    default: launch_attend<8>(grid, pow2, a, stream); break;
  }
  if (nsplit > 1)
    hipLaunchKernelGGL(attend_combine_kernel, dim3(R * H_q), dim3(kHeadDim), 0, stream,
                       reinterpret_cast<const float*>(ws), int(nsplit), out);
  return check_launch(nm);
}
