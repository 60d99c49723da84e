// Renormalised softmax attention over rows read by index (HashAttention
// study notes, sec. 2.1 sparse output formula; sec. 2.5 page-size-one reads:
// the selected rows are read in place by index, a 256-byte bf16 row being
// more than a cache line).  The matrix-core logits, the online softmax and
// the row fetch are in attend_dev.hpp; here a workgroup takes a run of a
// set's rows, each wave requests its next 32 rows before it works on the
// current 32, and sets split over several workgroups merge their partials by
// log-sum-exp rescaling in a second launch.
#include "attend_dev.hpp"

namespace sdq {

constexpr int kAtWaves = 4;
constexpr int kAtThreads = 64 * kAtWaves;
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

// Merges the nsplit partials of one query head (dim dd) in one pass with a
// running maximum, kCb partials at a time with each batch's loads issued
// together (one memory round trip per batch; the launch picks the smallest
// kCb of 4, 8 and 16 that covers nsplit, or 16, so a short merge issues no
// padding loads).
template <int kCb>
__device__ float merge_splits(const float* __restrict__ base, int nsplit, int dd) {
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
template <int CB>
__global__ __launch_bounds__(kHeadDim) void attend_combine_kernel(const float* __restrict__ parts,
                                                                  int nsplit,
                                                                  float* __restrict__ out) {
  const int qh = blockIdx.x, dd = threadIdx.x;
  out[size_t(qh) * kHeadDim + dd] =
      merge_splits<CB>(parts + size_t(qh) * nsplit * attend_partial_floats(kHeadDim), nsplit, dd);
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
  const AtSlices sl = at_slices(a.K, a.V, (size_t(r) * a.Hkv + kvh) * size_t(a.n_cap) * kHeadDim, a.n);

  // the query loads go out first, together with the idx loads of the row
  // offsets below
  float qv[4][8];
  at_load_q<NQ>(a.q + (size_t(r) * a.Hq + h0) * kHeadDim, qv);
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
  at_make_qf<NQ>(qv, qf);
  __syncthreads();

  // slab s of this wave: local rows (wave + s * W) * kAtSlab + ...
  const int my_slabs = wave < nslab ? (nslab - wave + W - 1) / W : 0;
  auto fetch = [&](int s, u32x4_t (&kw)[kAtGroups][4], u32x4_t (&vw)[kAtGroups][4],
                   uint32_t& vmask) {
    const bool live = s < my_slabs;           // past the wave's last slab: skipped rows
    at_fetch(sl, s_off + (wave + (live ? s : 0) * W) * kAtSlab, live, kw, vw, vmask);
  };
  AtState<NQ> st;
  at_init(st);

  // A wave with one slab requests it and works on it.  With more, two
  // register buffers: the next slab is requested before the current one is
  // used, in straight-line turns (slabs past the wave's last read as skipped
  // rows: no memory access, though their addresses still pass through the
  // CU's address unit; branching around them instead cost the long-set case
  // 3 % through the schedule of the loop).
  if (my_slabs == 1) {
    u32x4_t kA[kAtGroups][4], vA[kAtGroups][4];
    uint32_t mA;
    fetch(0, kA, vA, mA);
    at_compute<NQ>(st, qf, kA, vA, mA, a.scale_log2);
  } else if (my_slabs > 1) {
    u32x4_t kA[kAtGroups][4], vA[kAtGroups][4], kB[kAtGroups][4], vB[kAtGroups][4];
    uint32_t mA, mB;
    fetch(0, kA, vA, mA);
    for (int s = 0; s < my_slabs; s += 2) {
      fetch(s + 1, kB, vB, mB);
      at_compute<NQ>(st, qf, kA, vA, mA, a.scale_log2);
      fetch(s + 2, kA, vA, mA);
      if (s + 1 < my_slabs) at_compute<NQ>(st, qf, kB, vB, mB, a.scale_log2);
    }
  }

  // every lane row's state goes to LDS once all waves are done with the
  // offsets
  __syncthreads();
  float* sts = reinterpret_cast<float*>(s_lds);              // [kStates][NQ][d + 2]
  at_store_state<NQ>(st, sts, wave * 4 + g4);
  __syncthreads();
  // merge the states: one thread per (head, dim); write the output, or the
  // split's partial (unnormalised output, max in log2 units, sum)
  const size_t pf = attend_partial_floats(kHeadDim);
  for (int xi = tid; xi < NQ * kHeadDim; xi += kAtThreads) {
    const int h = xi / kHeadDim, dd = xi % kHeadDim;
    float Mx, L;
    const float acc = at_merge_states<NQ, kStates>(sts, h, dd, Mx, L);
    const size_t qh = size_t(r) * a.Hq + h0 + h;
    if (nsplit == 1) {
      a.out[qh * kHeadDim + dd] = (L > 0.0f) ? acc / L : 0.0f;
    } else {
      float* dst = a.parts + (qh * nsplit + split) * pf;
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
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(K) % 16 == 0 && reinterpret_cast<uintptr_t>(V) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(q) % 16 == 0,
              "%s: q, K and V must be 16-byte aligned", nm);
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
    hipLaunchKernelGGL(nsplit <= 4   ? attend_combine_kernel<4>
                       : nsplit <= 8 ? attend_combine_kernel<8>
                                     : attend_combine_kernel<16>,
                       dim3(R * H_q), dim3(kHeadDim), 0, stream,
                       reinterpret_cast<const float*>(ws), int(nsplit), out);
  return check_launch(nm);
}
