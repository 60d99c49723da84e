// Exact per-row top-k with lower-index tie-break and forced sink/local
// windows (HashAttention study notes, sec. 2.1 TOPK and sec. 3.1 fixed
// positions; OasisKV review, per-KV-head top-K over block summaries).
//
// Keys are mapped to order-preserving 32-bit codes u (float32: sign-folded
// bits, -0 first folded onto +0; uint8 distance d: 255 - d), so "best" is
// always "largest u", and ties go to the lower index.
//
// Two paths:
//  * row path (one workgroup per row): MSB-first radix select (8 bits per
//    pass, LDS histogram) finds the k-th largest code T and how many of the
//    codes equal to T to keep; a final pass walks the row in index order and
//    compacts the winners with block-wide prefix sums, so the output comes out
//    ascending with no sort.  Used for short rows, uint8 keys, and as the
//    fallback of the fast path.
//  * fast path for long float32 rows (many workgroups per row): one pass
//    builds a 2048-bin histogram of the top 11 bits of u, a tiny kernel picks
//    the bin holding the k-th code, a second pass appends every element of
//    that bin or above to a per-row candidate list, and one workgroup per row
//    selects exactly among the candidates (composite key (u, ~index) so every
//    key is distinct) and sorts the winners by index.  If the candidate list
//    overflows its capacity (heavily tied rows), that workgroup falls back to
//    the row path.
#include "common.hpp"

namespace sdq {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kFastMinComp = 65536;        // competition length that takes the fast path
constexpr int kHistBins = 2048;            // top 11 bits of the code
constexpr int kHistShift = 21;
constexpr int kCandCap = 8192;             // candidates per row
constexpr int kFastChunk = 4096;           // elements per workgroup in the fast passes

struct RowState {
  uint32_t bin;       // histogram bin holding the k-th code
  uint32_t count;     // candidates appended (may exceed the capacity)
  uint32_t pad[14];
};

__host__ __device__ inline size_t fast_ws_per_row() {
  return size_t(kHistBins) * 4 + sizeof(RowState) + size_t(kCandCap) * 8;
}

template <int KT>
__device__ __forceinline__ uint32_t load_code(const void* __restrict__ keys, size_t i) {
  if (KT == SDQ_KEY_F32_MAX) return f32_order_key(reinterpret_cast<const float*>(keys)[i]);
  return 255u - reinterpret_cast<const uint8_t*>(keys)[i];
}

// Block-wide exclusive prefix sums of two counters (512 threads).
__device__ __forceinline__ void block_scan2(int a, int b, int& ea, int& eb, int& ta, int& tb,
                                            int* s_scan) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int x = __shfl_up(ia, off, 64), y = __shfl_up(ib, off, 64);
    if (lane >= off) {
      ia += x;
      ib += y;
    }
  }
  if (lane == 63) {
    s_scan[wave] = ia;
    s_scan[kTkWaves + wave] = ib;
  }
  __syncthreads();
  int wa = 0, wb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const int va = s_scan[w], vb = s_scan[kTkWaves + w];
    if (w < wave) {
      wa += va;
      wb += vb;
    }
    ta += va;
    tb += vb;
  }
  ea = wa + ia - a;
  eb = wb + ib - b;
  __syncthreads();
}

// Writes the fixed positions and padding of one output row.
__device__ __forceinline__ void write_fixed(int32_t* o, int n, int n_sink, int n_local, int K,
                                            int stride) {
  const int hi = n - n_local;
  for (int i = threadIdx.x; i < n_sink; i += blockDim.x) o[i] = i;
  for (int i = threadIdx.x; i < n_local; i += blockDim.x) o[n_sink + K + i] = hi + i;
  for (int i = n_sink + K + n_local + threadIdx.x; i < stride; i += blockDim.x) o[i] = -1;
}

// The row path for one row; all threads of the workgroup call it.
template <int KT>
__device__ void topk_row(const void* __restrict__ keys, size_t base, int n, int k, int n_sink,
                         int n_local, int32_t* __restrict__ o, int stride) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_need;
  __shared__ int s_scan[2 * kTkWaves];
  const int tid = threadIdx.x;
  const int lo = n_sink, hi = n - n_local, m = hi - lo;
  const int K = k < m ? k : m;
  write_fixed(o, n, n_sink, n_local, K, stride);
  if (K == m) {
    for (int i = tid; i < m; i += kTkThreads) o[n_sink + i] = lo + i;
    return;
  }
  if (K == 0) return;

  uint32_t prefix = 0, pmask = 0;
  int need = K;
  const int first_shift = (KT == SDQ_KEY_U8_MIN) ? 0 : 24;
  for (int shift = first_shift; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = lo + tid; i < hi; i += kTkThreads) {
      const uint32_t u = load_code<KT>(keys, base + i);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // suffix sums over the 256 bins; lane l owns bins 4l..4l+3
      const int l = tid;
      const int c0 = hist[4 * l], c1 = hist[4 * l + 1], c2 = hist[4 * l + 2], c3 = hist[4 * l + 3];
      const int lsum = c0 + c1 + c2 + c3;
      int sfx = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_down(sfx, off, 64);
        if (l + off < 64) sfx += y;
      }
      const int above = sfx - lsum;               // codes in higher lanes' bins
      const int S3 = above + c3, S2 = S3 + c2, S1 = S2 + c1, S0 = S1 + c0;
      if (S3 >= need && above < need) { sh_digit = 4 * l + 3; sh_need = need - above; }
      if (S2 >= need && S3 < need) { sh_digit = 4 * l + 2; sh_need = need - S3; }
      if (S1 >= need && S2 < need) { sh_digit = 4 * l + 1; sh_need = need - S2; }
      if (S0 >= need && S1 < need) { sh_digit = 4 * l; sh_need = need - S1; }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    need = sh_need;
    __syncthreads();
  }
  const uint32_t T = prefix;       // k-th largest code; keep every u > T and the first `need` u == T

  constexpr int IPT = 8;
  int out_pos = n_sink, eq_seen = 0;
  for (int c0 = lo; c0 < hi; c0 += kTkThreads * IPT) {
    const int i0 = c0 + tid * IPT;
    uint32_t u[IPT];
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      const int i = i0 + e;
      u[e] = (i < hi) ? load_code<KT>(keys, base + i) : 0u;
      if (i < hi) {
        gt += u[e] > T;
        eq += u[e] == T;
      }
    }
    int egt, eeq, tgt, teq;
    block_scan2(gt, eq, egt, eeq, tgt, teq, s_scan);
    const int eq_left = need - eq_seen > 0 ? need - eq_seen : 0;
    int pos = out_pos + egt + (eeq < eq_left ? eeq : eq_left);
    int my_eq = eeq;
    const int end = n_sink + K;              // never write past the selected range
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      const int i = i0 + e;
      if (i < hi) {
        if (u[e] > T) {
          if (pos < end) o[pos] = i;
          ++pos;
        } else if (u[e] == T) {
          if (my_eq < eq_left) {
            if (pos < end) o[pos] = i;
            ++pos;
          }
          ++my_eq;
        }
      }
    }
    out_pos += tgt + (teq < eq_left ? teq : eq_left);
    eq_seen += teq;
  }
}

template <int KT>
__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(const void* __restrict__ keys, int n,
                                                              int k, int n_sink, int n_local,
                                                              int32_t* __restrict__ out,
                                                              int stride) {
  const int row = blockIdx.x;
  topk_row<KT>(keys, size_t(row) * n, n, k, n_sink, n_local, out + size_t(row) * stride, stride);
}

// ------------------------------------------------------------- fast path
__device__ __forceinline__ uint32_t* ws_hist(void* ws, int row) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + size_t(row) * fast_ws_per_row());
}
__device__ __forceinline__ RowState* ws_state(void* ws, int row) {
  return reinterpret_cast<RowState*>(ws_hist(ws, row) + kHistBins);
}
__device__ __forceinline__ uint2* ws_cand(void* ws, int row) {
  return reinterpret_cast<uint2*>(ws_state(ws, row) + 1);
}

__global__ __launch_bounds__(256) void topk_clear_kernel(void* ws) {
  uint32_t* h = ws_hist(ws, blockIdx.x);
  for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0;
  if (threadIdx.x == 0) {
    RowState* s = ws_state(ws, blockIdx.x);
    s->bin = 0;
    s->count = 0;
  }
}

__global__ __launch_bounds__(256) void topk_hist_kernel(const float* __restrict__ keys, int n, int lo,
                                                        int hi, void* ws) {
  __shared__ uint32_t h[kHistBins];
  const int row = blockIdx.y;
  for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0;
  __syncthreads();
  const size_t base = size_t(row) * n;
  const int c0 = lo + blockIdx.x * kFastChunk;
  for (int e = 0; e < kFastChunk / 256; ++e) {
    const int i = c0 + e * 256 + threadIdx.x;
    if (i < hi) atomicAdd(&h[f32_order_key(keys[base + i]) >> kHistShift], 1u);
  }
  __syncthreads();
  uint32_t* gh = ws_hist(ws, row);
  for (int i = threadIdx.x; i < kHistBins; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// One workgroup (256 threads) per row: the bin that holds the K-th code.
__global__ __launch_bounds__(256) void topk_bin_kernel(void* ws, int K) {
  __shared__ int s_part[256];
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint32_t* gh = ws_hist(ws, row);
  // thread t owns bins 8t..8t+7
  int c[8], tot = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    c[e] = int(gh[8 * tid + e]);
    tot += c[e];
  }
  s_part[tid] = tot;
  __syncthreads();
  int above = 0;                       // codes in bins of higher threads
  for (int t = tid + 1; t < 256; ++t) above += s_part[t];
  int S_next = above;                  // codes in bins above the current one
#pragma unroll
  for (int e = 7; e >= 0; --e) {
    const int S = S_next + c[e];
    if (S >= K && S_next < K) ws_state(ws, row)->bin = uint32_t(8 * tid + e);
    S_next = S;
  }
}

__global__ __launch_bounds__(256) void topk_collect_kernel(const float* __restrict__ keys, int n,
                                                           int lo, int hi, void* ws) {
  const int row = blockIdx.y;
  RowState* st = ws_state(ws, row);
  uint2* cand = ws_cand(ws, row);
  const uint32_t bin = st->bin;
  const size_t base = size_t(row) * n;
  const int c0 = lo + blockIdx.x * kFastChunk;
  for (int e = 0; e < kFastChunk / 256; ++e) {
    const int i = c0 + e * 256 + threadIdx.x;
    uint32_t u = 0;
    bool keep = false;
    if (i < hi) {
      u = f32_order_key(keys[base + i]);
      keep = (u >> kHistShift) >= bin;
    }
    // one atomic per wave for the wave's candidates
    const uint64_t mask = __ballot(keep);
    if (mask) {
      const int lane = threadIdx.x & 63;
      const int leader = __ffsll((unsigned long long)mask) - 1;
      uint32_t slot0 = 0;
      if (lane == leader) slot0 = atomicAdd(&st->count, uint32_t(__popcll(mask)));
      slot0 = __shfl(slot0, leader, 64);
      if (keep) {
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const uint32_t slot = slot0 + uint32_t(__popcll(mask & lt));
        if (slot < uint32_t(kCandCap)) cand[slot] = make_uint2(u, uint32_t(i));
      }
    }
  }
}

// One workgroup per row: exact selection among the candidates, then sort the
// winners by index.  Falls back to the row path when the list overflowed.
__global__ __launch_bounds__(kTkThreads) void topk_final_kernel(const float* __restrict__ keys,
                                                                int n, int k, int n_sink,
                                                                int n_local, void* ws,
                                                                int32_t* __restrict__ out,
                                                                int stride) {
  __shared__ uint64_t ck[kCandCap];       // composite keys (u << 32) | ~index
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_need;
  __shared__ int sh_cnt;
  const int row = blockIdx.x, tid = threadIdx.x;
  int32_t* o = out + size_t(row) * stride;
  const uint32_t count = ws_state(ws, row)->count;
  const int lo = n_sink, hi = n - n_local, m = hi - lo;
  const int K = k < m ? k : m;
  if (count > uint32_t(kCandCap) || K > kCandCap) {
    topk_row<SDQ_KEY_F32_MAX>(keys, size_t(row) * n, n, k, n_sink, n_local, o, stride);
    return;
  }
  write_fixed(o, n, n_sink, n_local, K, stride);
  const int cnt = int(count);
  const uint2* cand = ws_cand(ws, row);
  for (int i = tid; i < cnt; i += kTkThreads) {
    const uint2 c = cand[i];
    ck[i] = (uint64_t(c.x) << 32) | uint64_t(~c.y);
  }
  __syncthreads();
  // radix select of the K-th largest composite key (all distinct)
  uint64_t prefix = 0, pmask = 0;
  int need = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < cnt; i += kTkThreads) {
      const uint64_t v = ck[i];
      if ((v & pmask) == prefix) atomicAdd(&hist[uint32_t(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const int l = tid;
      const int c0 = hist[4 * l], c1 = hist[4 * l + 1], c2 = hist[4 * l + 2], c3 = hist[4 * l + 3];
      const int lsum = c0 + c1 + c2 + c3;
      int sfx = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_down(sfx, off, 64);
        if (l + off < 64) sfx += y;
      }
      const int above = sfx - lsum;
      const int S3 = above + c3, S2 = S3 + c2, S1 = S2 + c1, S0 = S1 + c0;
      if (S3 >= need && above < need) { sh_digit = 4 * l + 3; sh_need = need - above; }
      if (S2 >= need && S3 < need) { sh_digit = 4 * l + 2; sh_need = need - S3; }
      if (S1 >= need && S2 < need) { sh_digit = 4 * l + 1; sh_need = need - S2; }
      if (S0 >= need && S1 < need) { sh_digit = 4 * l; sh_need = need - S1; }
    }
    __syncthreads();
    prefix |= uint64_t(sh_digit) << shift;
    pmask |= uint64_t(255) << shift;
    need = sh_need;
    __syncthreads();
  }
  // winners: composite >= prefix (exactly K of them); gather their indices
  __shared__ int widx[kCandCap];
  if (tid == 0) sh_cnt = 0;
  __syncthreads();
  for (int i = tid; i < cnt; i += kTkThreads) {
    const uint64_t v = ck[i];
    if (v >= prefix) widx[atomicAdd(&sh_cnt, 1)] = int(~uint32_t(v));
  }
  __syncthreads();
  int P = 1;
  while (P < K) P <<= 1;
  for (int i = K + tid; i < P; i += kTkThreads) widx[i] = 0x7FFFFFFF;
  __syncthreads();
  // bitonic sort of P indices, ascending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride2 = size >> 1; stride2 > 0; stride2 >>= 1) {
      for (int t = tid; t < P / 2; t += kTkThreads) {
        const int i = 2 * t - (t & (stride2 - 1));
        const int j = i + stride2;
        const bool up = (i & size) == 0;
        const int a = widx[i], b = widx[j];
        if ((a > b) == up) {
          widx[i] = b;
          widx[j] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < K; i += kTkThreads) o[n_sink + i] = widx[i];
}

}  // namespace sdq

using namespace sdq;

static bool use_fast(int n, int n_sink, int n_local, int k, int key_type) {
  const int m = n - n_sink - n_local;
  return key_type == SDQ_KEY_F32_MAX && m >= kFastMinComp && k < m && k <= kCandCap;
}

extern "C" size_t topk_select_workspace_bytes(int rows, int n, int k, int key_type) {
  if (rows < 1 || n < 1) return 0;
  (void)k;
  if (key_type == SDQ_KEY_F32_MAX && n >= kFastMinComp) return size_t(rows) * fast_ws_per_row();
  return 256;
}

extern "C" int topk_select(const void* keys, int key_type, int rows, int n, int k, int n_sink,
                           int n_local, int32_t* idx_out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  SDQ_REQUIRE(keys && idx_out, "topk_select: null pointer");
  SDQ_REQUIRE(key_type == SDQ_KEY_F32_MAX || key_type == SDQ_KEY_U8_MIN,
              "topk_select: unknown key_type %d", key_type);
  SDQ_REQUIRE(rows >= 1 && n >= 1, "topk_select: rows=%d, n=%d must be >= 1", rows, n);
  SDQ_REQUIRE(k >= 0 && n_sink >= 0 && n_local >= 0, "topk_select: k, n_sink, n_local must be >= 0");
  SDQ_REQUIRE(n_sink <= n - n_local, "topk_select: n_sink + n_local = %d exceeds n = %d",
              n_sink + n_local, n);
  const long long stride_ll = (long long)k + n_sink + n_local;
  SDQ_REQUIRE(stride_ll <= 0x7FFFFFFF, "topk_select: output row too long");
  const int stride = int(stride_ll);
  const size_t need_ws = topk_select_workspace_bytes(rows, n, k, key_type);
  if (stride == 0) return SDQ_OK;
  if (use_fast(n, n_sink, n_local, k, key_type)) {
    SDQ_REQUIRE(ws && ws_bytes >= need_ws, "topk_select: workspace of %zu bytes needed, %zu given",
                need_ws, ws_bytes);
    const int lo = n_sink, hi = n - n_local;
    const float* fk = reinterpret_cast<const float*>(keys);
    dim3 g2(cdiv(hi - lo, kFastChunk), rows);
    hipLaunchKernelGGL(topk_clear_kernel, dim3(rows), dim3(256), 0, stream, ws);
    hipLaunchKernelGGL(topk_hist_kernel, g2, dim3(256), 0, stream, fk, n, lo, hi, ws);
    const int K = k;
    hipLaunchKernelGGL(topk_bin_kernel, dim3(rows), dim3(256), 0, stream, ws, K);
    hipLaunchKernelGGL(topk_collect_kernel, g2, dim3(256), 0, stream, fk, n, lo, hi, ws);
    hipLaunchKernelGGL(topk_final_kernel, dim3(rows), dim3(kTkThreads), 0, stream, fk, n, k, n_sink,
                       n_local, ws, idx_out, stride);
    return check_launch("topk_select");
  }
  if (key_type == SDQ_KEY_F32_MAX)
    hipLaunchKernelGGL(topk_row_kernel<SDQ_KEY_F32_MAX>, dim3(rows), dim3(kTkThreads), 0, stream,
                       keys, n, k, n_sink, n_local, idx_out, stride);
  else
    hipLaunchKernelGGL(topk_row_kernel<SDQ_KEY_U8_MIN>, dim3(rows), dim3(kTkThreads), 0, stream,
                       keys, n, k, n_sink, n_local, idx_out, stride);
  return check_launch("topk_select");
}
