// Renormalised softmax attention over rows read by index (HashAttention
// study notes, sec. 2.1 sparse output formula; sec. 2.5 page-size-one reads:
// the selected rows are read in place by index, a 256-byte bf16 row being
// more than a cache line).
//
// Split over row chunks: each workgroup takes CH selected rows of one set
// and all query heads that share the set (the GQA group, or one head), and
// writes a partial (max logit m, sum of exponentials l, unnormalised output
// o); a combine kernel merges the chunks of every query head with the usual
// log-sum-exp rescaling.  Inside a chunk, 16 lanes share a row (8 dims each,
// one 16-byte load of K and one of V), so a 256-thread workgroup handles 16
// rows per step; every K/V row is read once for all the group's heads.
// fp32 arithmetic throughout.
#include "common.hpp"

namespace sdq {

constexpr int kAtThreads = 256;
constexpr int kAtChunk = 64;            // selected rows per workgroup
constexpr int kAtRowsPerStep = kAtThreads / 16;

struct AttendArgs {
  const float* q;
  const uint4* K;
  const uint4* V;
  const int32_t* idx;
  int R, Hq, Hkv, per_qh, n, n_idx, bt, nchunks;
  float scale;
  float* ws;
};

__host__ __device__ inline size_t attend_partial_floats(int d) { return size_t(d) + 2; }

template <int NQ>
__global__ __launch_bounds__(kAtThreads) void attend_partial_kernel(AttendArgs a) {
  __shared__ int tok[kAtChunk];
  __shared__ float z[kAtChunk][NQ];
  __shared__ float s_m[NQ], s_l[NQ];
  __shared__ float red[kAtThreads / 64][NQ][kHeadDim];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = tid & 15;                 // dims 8*sub .. 8*sub+7
  const int rslot = tid >> 4;               // row slot within a step (0..15)
  const int chunk = blockIdx.x;
  const int set = blockIdx.y;               // r * Hsel + hs
  const int Hsel = a.per_qh ? a.Hq : a.Hkv;
  const int r = set / Hsel, hs = set % Hsel;
  const int grp = a.Hq / a.Hkv;
  const int kvh = a.per_qh ? hs / grp : hs;
  const int h0 = a.per_qh ? hs : hs * grp;  // first query head of the set
  const int M = a.n_idx * a.bt;

  for (int i = tid; i < kAtChunk; i += kAtThreads) {
    const int row = chunk * kAtChunk + i;
    int t = -1;
    if (row < M) {
      const int e = a.idx[size_t(set) * a.n_idx + row / a.bt];
      if (e >= 0) {
        const long long tt = (long long)e * a.bt + row % a.bt;
        t = tt < a.n ? int(tt) : -1;
      }
    }
    tok[i] = t;
  }
  float qr[NQ][8];
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    const float* qp = a.q + (size_t(r) * a.Hq + h0 + h) * kHeadDim + 8 * sub;
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[h][e] = qp[e];
  }
  __syncthreads();

  const size_t kvbase = (size_t(r) * a.Hkv + kvh) * size_t(a.n);
  // every K and V row of the chunk is requested before any arithmetic, so the
  // chunk costs one memory round trip
  constexpr int kSteps = kAtChunk / kAtRowsPerStep;
  uint4 kw[kSteps], vw[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int t = tok[s * kAtRowsPerStep + rslot];
    const size_t off = (kvbase + (t >= 0 ? t : 0)) * (kHeadDim / 8) + sub;
    kw[s] = t >= 0 ? a.K[off] : make_uint4(0u, 0u, 0u, 0u);
    vw[s] = t >= 0 ? a.V[off] : make_uint4(0u, 0u, 0u, 0u);
  }
  // logits
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int i = s * kAtRowsPerStep + rslot;
    const int t = tok[i];
    const float kf[8] = {bf16_lo(kw[s].x), bf16_hi(kw[s].x), bf16_lo(kw[s].y), bf16_hi(kw[s].y),
                         bf16_lo(kw[s].z), bf16_hi(kw[s].z), bf16_lo(kw[s].w), bf16_hi(kw[s].w)};
    float part[NQ];
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      part[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part[h] = __builtin_fmaf(qr[h][e], kf[e], part[h]);
    }
#pragma unroll
    for (int h = 0; h < NQ; ++h) part[h] = row16_sum(part[h]);   // over the row's 16 lanes
    if (sub == 0) {
#pragma unroll
      for (int h = 0; h < NQ; ++h) z[i][h] = (t >= 0) ? part[h] * a.scale : -INFINITY;
    }
  }
  __syncthreads();
  // softmax statistics per head: one wave per head
  for (int h = wave; h < NQ; h += kAtThreads / 64) {
    float mx = -INFINITY;
    for (int i = lane; i < kAtChunk; i += 64) mx = fmaxf(mx, z[i][h]);
    mx = wave_max_f32(mx);
    float l = 0.0f;
    for (int i = lane; i < kAtChunk; i += 64) {
      const float p = (mx == -INFINITY) ? 0.0f : __expf(z[i][h] - mx);
      z[i][h] = p;
      l += p;
    }
    l = wave_sum_f32(l);
    if (lane == 0) {
      s_m[h] = mx;
      s_l[h] = l;
    }
  }
  __syncthreads();
  // weighted values
  float o[NQ][8];
#pragma unroll
  for (int h = 0; h < NQ; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int i = s * kAtRowsPerStep + rslot;
    const float vf[8] = {bf16_lo(vw[s].x), bf16_hi(vw[s].x), bf16_lo(vw[s].y), bf16_hi(vw[s].y),
                         bf16_lo(vw[s].z), bf16_hi(vw[s].z), bf16_lo(vw[s].w), bf16_hi(vw[s].w)};
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      const float p = z[i][h];                  // 0 for skipped rows
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = __builtin_fmaf(p, vf[e], o[h][e]);
    }
  }
  // reduce the 4 row slots of a wave (lanes sub, sub+16, sub+32, sub+48)
#pragma unroll
  for (int h = 0; h < NQ; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[h][e] += __shfl_xor(o[h][e], 16, 64);
      o[h][e] += __shfl_xor(o[h][e], 32, 64);
    }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < NQ; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][h][8 * sub + e] = o[h][e];
  }
  __syncthreads();
  // across waves, then write the partial of every head of the set
  const size_t pf = attend_partial_floats(kHeadDim);
  for (int x = tid; x < NQ * kHeadDim; x += kAtThreads) {
    const int h = x / kHeadDim, dd = x % kHeadDim;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kAtThreads / 64; ++w) acc += red[w][h][dd];
    const size_t qh = size_t(r) * a.Hq + h0 + h;
    float* dst = a.ws + (qh * a.nchunks + chunk) * pf;
    dst[dd] = acc;
    if (dd == 0) {
      dst[kHeadDim] = s_m[h];
      dst[kHeadDim + 1] = s_l[h];
    }
  }
}

// One workgroup per query head: merges the chunks' partials, kCb chunks per
// batch with all of a batch's loads issued together.
__global__ __launch_bounds__(kHeadDim) void attend_combine_kernel(const float* __restrict__ ws,
                                                                  int nchunks,
                                                                  float* __restrict__ out) {
  constexpr int kCb = 16;
  const int qh = blockIdx.x, dd = threadIdx.x;
  const size_t pf = attend_partial_floats(kHeadDim);
  const float* base = ws + size_t(qh) * nchunks * pf;
  float M = -INFINITY;
  for (int c0 = 0; c0 < nchunks; c0 += kCb) {
    float mv[kCb];
#pragma unroll
    for (int e = 0; e < kCb; ++e) mv[e] = c0 + e < nchunks ? base[(c0 + e) * pf + kHeadDim] : -INFINITY;
#pragma unroll
    for (int e = 0; e < kCb; ++e) M = fmaxf(M, mv[e]);
  }
  float L = 0.0f, acc = 0.0f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < nchunks; c0 += kCb) {
      float mv[kCb], lv[kCb], ov[kCb];
#pragma unroll
      for (int e = 0; e < kCb; ++e) {
        const bool in = c0 + e < nchunks;
        const float* pc = base + (in ? c0 + e : 0) * pf;
        mv[e] = in ? pc[kHeadDim] : -INFINITY;
        lv[e] = pc[kHeadDim + 1];
        ov[e] = pc[dd];
      }
#pragma unroll
      for (int e = 0; e < kCb; ++e) {
        const float w = (mv[e] == -INFINITY) ? 0.0f : __expf(mv[e] - M);
        L = __builtin_fmaf(lv[e], w, L);
        acc = __builtin_fmaf(ov[e], w, acc);
      }
    }
  }
  out[size_t(qh) * kHeadDim + dd] = (L > 0.0f) ? acc / L : 0.0f;
}

}  // namespace sdq

using namespace sdq;

static int attend_nchunks(int n_idx, int bt) {
  const long long M = (long long)n_idx * bt;
  return int((M + kAtChunk - 1) / kAtChunk);
}

extern "C" size_t gather_attend_workspace_bytes(int R, int H_q, int H_kv, int sets_per_query_head,
                                                int n_idx, int block_tokens, int d) {
  (void)H_kv;
  (void)sets_per_query_head;
  if (R < 1 || H_q < 1 || n_idx < 1 || block_tokens < 1 || d != kHeadDim) return 0;
  return size_t(R) * H_q * attend_nchunks(n_idx, block_tokens) * attend_partial_floats(d) *
         sizeof(float);
}

extern "C" int gather_attend(const float* q, const uint16_t* K, const uint16_t* V,
                             const int32_t* idx, int R, int H_q, int H_kv, int sets_per_query_head,
                             int n, int n_idx, int block_tokens, int d, float softmax_scale,
                             float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  SDQ_REQUIRE(q && K && V && idx && out, "gather_attend: null pointer");
  SDQ_REQUIRE(R >= 1 && H_q >= 1 && H_kv >= 1 && n >= 1 && n_idx >= 1 && block_tokens >= 1,
              "gather_attend: R, H_q, H_kv, n, n_idx, block_tokens must be >= 1");
  SDQ_REQUIRE(H_q % H_kv == 0, "gather_attend: H_q=%d not a multiple of H_kv=%d", H_q, H_kv);
  SDQ_REQUIRE(d == kHeadDim, "gather_attend: d=%d unsupported (only 128)", d);
  SDQ_REQUIRE((long long)n_idx * block_tokens <= 0x7FFFFFFFLL, "gather_attend: too many rows");
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(K) % 16 == 0 && reinterpret_cast<uintptr_t>(V) % 16 == 0,
              "gather_attend: K and V must be 16-byte aligned");
  const int grp = H_q / H_kv;
  const int NQ = sets_per_query_head ? 1 : grp;
  SDQ_REQUIRE(NQ == 1 || NQ == 2 || NQ == 4 || NQ == 8,
              "gather_attend: %d query heads per set unsupported (1, 2, 4 or 8)", NQ);
  const size_t need = gather_attend_workspace_bytes(R, H_q, H_kv, sets_per_query_head, n_idx,
                                                    block_tokens, d);
  SDQ_REQUIRE(ws && ws_bytes >= need, "gather_attend: workspace of %zu bytes needed, %zu given",
              need, ws_bytes);
  const int nchunks = attend_nchunks(n_idx, block_tokens);
  const int Hsel = sets_per_query_head ? H_q : H_kv;
  AttendArgs a{q, reinterpret_cast<const uint4*>(K), reinterpret_cast<const uint4*>(V), idx, R, H_q,
               H_kv, sets_per_query_head ? 1 : 0, n, n_idx, block_tokens, nchunks, softmax_scale,
               reinterpret_cast<float*>(ws)};
  dim3 grid(nchunks, R * Hsel);
  switch (NQ) {
    case 1: hipLaunchKernelGGL(attend_partial_kernel<1>, grid, dim3(kAtThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(attend_partial_kernel<2>, grid, dim3(kAtThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(attend_partial_kernel<4>, grid, dim3(kAtThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL(attend_partial_kernel<8>, grid, dim3(kAtThreads), 0, stream, a); break;
  }
  hipLaunchKernelGGL(attend_combine_kernel, dim3(R * H_q), dim3(kHeadDim), 0, stream,
                     reinterpret_cast<const float*>(ws), nchunks, out);
  return check_launch("gather_attend");
}
