// Exact per-row top-k with lower-index tie-break and forced sink/local
// windows (HashAttention study notes, sec. 2.1 TOPK and sec. 3.1 fixed
// positions; OasisKV review, per-KV-head top-K over block summaries).
//
// Keys are mapped to order-preserving 32-bit codes u (float32: sign-folded
// bits, -0 first folded onto +0; uint8 distance d: 255 - d), so "best" is
// always "largest u", and ties go to the lower index.
//
// Paths:
//  * row path (one workgroup per row): MSB-first radix select (8 bits per
//    pass, LDS histogram) finds the k-th largest code T and how many of the
//    codes equal to T to keep; a final pass walks the row in index order and
//    compacts the winners with block-wide prefix sums, so the output comes out
//    ascending with no sort.  Used for float32 rows of at most 1024 keys and
//    as the fallback of the other paths.
//  * register row path (one workgroup per row, 1025..32768 float32 keys):
//    the row is read once into registers, in an order where wave ballots give
//    index order, and the histogram, candidate and winner passes work on the
//    registers (see topk_row_reg_kernel).
//  * uint8 paths: one 256-bin histogram settles the select in a single pass
//    (one workgroup per row), or, for long rows, per-segment histograms in
//    the workspace let one workgroup per segment place its own winners.
//  * block-max path (topk_select_block_max): float32 rows whose 64-key block
//    maxima are known read only the blocks that can hold a winner.  Its split
//    form (topk_select_block_max_split) spreads each row's candidate gather
//    over several workgroups and selects in a second launch.
//  * fast path for long float32 rows (many workgroups per row): one pass
//    builds a 2048-bin histogram of the top 11 bits of u, a tiny kernel picks
//    the bin holding the k-th code, a second pass appends every element of
//    that bin or above to a per-row candidate list, and one workgroup per row
//    selects exactly among the candidates (composite key (u, ~index) so every
//    key is distinct) and sorts the winners by index.  If the candidate list
//    overflows its capacity (heavily tied rows), that workgroup falls back to
//    the row path.
#include "common.hpp"

#include <mutex>

namespace sdq {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kFastMinComp = 32769;        // competition length that takes the fast path
constexpr int kBmMinComp = 65536;          // ... and the block-max path
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

// Block-wide exclusive prefix sums of two counters (512 threads).  With
// kTail = false the closing barrier is left out: the caller must pass a
// barrier (or use another s_scan buffer) before s_scan is written again.
template <bool kTail = true>
__device__ __forceinline__ void block_scan2(int a, int b, int& ea, int& eb, int& ta, int& tb,
                                            int* s_scan) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
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
  if (kTail) __syncthreads();
}

// Block-wide exclusive prefix sum of one counter (512 threads).
template <bool kTail = true>
__device__ __forceinline__ int block_scan1(int a, int& total, int* s_scan) {
  int ea, eb, tb;
  block_scan2<kTail>(a, 0, ea, eb, total, tb, s_scan);
  return ea;
}

// k-th largest of a set of 32-bit codes, for a whole 512-thread workgroup.
// fetch(i, &u) returns false for items that do not take part.  Each pass
// histograms the codes inside the current range [lo, hi] into 256 bins of
// width 2^s chosen so the bins span the range (bins follow the data, so
// clustered codes do not pile onto one LDS counter), then narrows the range
// to the bin holding the k-th code.  Returns the code T and how many of the
// codes equal to T belong to the top k (`need`).
//
// One barrier per pass: the passes rotate over three histograms (kKthHist
// words of LDS), a pass clears the one two passes ahead after its barrier,
// and every wave finds the k-th bin by itself (four bins a lane and a wave
// prefix sum), so no result travels through LDS.  Histograms 0 and 1 must be
// zero on entry to select_kth_in (select_kth clears them); the function ends
// with a barrier, so hist and s_red are free again on return.
constexpr int kKthHist = 3 * 256;

struct KthResult {
  uint32_t T;
  int need;
};

template <typename Fetch>
__device__ KthResult select_kth_in(int count, int K, Fetch fetch, uint32_t* hist, uint32_t lo,
                                   uint32_t hi) {
  const int tid = threadIdx.x, lane = tid & 63;
  int need = K;
  for (int p = 0; lo < hi; ++p) {
    const uint32_t width = hi - lo;
    const int bits = 32 - __clz(width);                 // width < 2^bits
    const int sh = bits > 8 ? bits - 8 : 0;              // (width >> sh) < 256
    uint32_t* h = hist + 256 * (p % 3);
    for (int i = tid; i < count; i += kTkThreads) {
      uint32_t u;
      if (fetch(i, &u) && u >= lo && u <= hi) atomicAdd(&h[(u - lo) >> sh], 1u);
    }
    __syncthreads();
    // the histogram of pass p + 2 was last read before this barrier
    if (tid < 256) hist[256 * ((p + 2) % 3) + tid] = 0;
    const uint4 c = *reinterpret_cast<const uint4*>(h + 4 * lane);
    const int lsum = int(c.x + c.y + c.z + c.w);
    const int inc = wave_incl_scan(lsum);
    const int above = wave_last(inc) - inc;             // counts in higher lanes' bins
    const int S3 = above + int(c.w), S2 = S3 + int(c.z), S1 = S2 + int(c.y);
    // the one lane whose bins take the count from below `need` to `need` or more
    const uint64_t hit = __ballot(above < need && above + lsum >= need);
    const int L = __ffsll((unsigned long long)hit) - 1;
    int d, rest;
    if (S3 >= need) { d = 3; rest = need - above; }
    else if (S2 >= need) { d = 2; rest = need - S3; }
    else if (S1 >= need) { d = 1; rest = need - S2; }
    else { d = 0; rest = need - S1; }
    const uint32_t bin = uint32_t(4 * L + __builtin_amdgcn_readlane(d, L));
    need = __builtin_amdgcn_readlane(rest, L);
    const uint32_t nlo = lo + (bin << sh);
    const uint32_t span = (sh >= 32) ? 0xFFFFFFFFu : ((1u << sh) - 1u);
    hi = (hi - nlo) > span ? nlo + span : hi;
    lo = nlo;
  }
  __syncthreads();
  return KthResult{lo, need};
}

template <typename Fetch>
__device__ KthResult select_kth(int count, int K, Fetch fetch, uint32_t* hist, uint32_t* s_red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // range of the codes
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = tid; i < count; i += kTkThreads) {
    uint32_t u;
    if (fetch(i, &u)) {
      mn = u < mn ? u : mn;
      mx = u > mx ? u : mx;
    }
  }
  mn = wave_minmax_u32<false>(mn);
  mx = wave_minmax_u32<true>(mx);
  if (lane == 0) {
    s_red[wave] = mn;
    s_red[kTkWaves + wave] = mx;
  }
  for (int i = tid; i < 2 * 256; i += kTkThreads) hist[i] = 0;
  __syncthreads();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    lo = s_red[w] < lo ? s_red[w] : lo;
    hi = s_red[kTkWaves + w] > hi ? s_red[kTkWaves + w] : hi;
  }
  return select_kth_in(count, K, fetch, hist, lo, hi);
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
  __shared__ __align__(16) uint32_t hist[kKthHist];
  __shared__ int s_scan[4 * kTkWaves];    // two buffers: the chunk scans alternate
  const int tid = threadIdx.x;
  const int lo = n_sink, hi = n - n_local, m = hi - lo;
  const int K = k < m ? k : m;
  write_fixed(o, n, n_sink, n_local, K, stride);
  if (K == m) {
    for (int i = tid; i < m; i += kTkThreads) o[n_sink + i] = lo + i;
    return;
  }
  if (K == 0) return;

  __shared__ uint32_t s_red[2 * kTkWaves];
  const KthResult kr = select_kth(
      m, K,
      [&](int i, uint32_t* u) {
        *u = load_code<KT>(keys, base + lo + i);
        return true;
      },
      hist, s_red);
  const uint32_t T = kr.T;         // k-th largest code; keep every u > T and the first `need` u == T
  const int need = kr.need;

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
    block_scan2<false>(gt, eq, egt, eeq, tgt, teq,
                       s_scan + 2 * kTkWaves * (((c0 - lo) / (kTkThreads * IPT)) & 1));
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

// Rows of at most CAP competing float32 keys are read from memory once, into
// registers, and every later pass works on them.  Wave w holds the 64 PER
// consecutive keys from 64 PER w on, lane l the keys 64 PER w + 64 e + l for
// e < PER: a wave's loads are contiguous, and (wave, e, lane) is index order,
// so wave ballots give in-order positions without an LDS copy of the row:
//  1. order-preserving codes into registers (every load in flight together)
//     and their range;
//  2. a 4096-bin LDS histogram over the range; the bin b* holding the K-th
//     largest code;
//  3. the codes of bin b* compacted into a short LDS list in index order
//     (per-wave ballot counts, one barrier for the wave offsets);
//  4. the exact K-th code T and how many of its ties to keep, among them;
//  5. the winners written in index order: the ballots of "above T" and
//     "equal to T" for every (wave, e) go to two LDS bitmaps (lane e of the
//     wave collects word e), then thread t takes bitmap word t, one prefix sum
//     over the words places its winners, and the first `need` ties in index
//     order are kept.
// Slots past the row end (the last PER*512 - m in index order) hold copies of
// the row's last key, so no pass needs a validity mask: the histogram and the
// candidate count take the copies back out, and coming last in index order
// they never take an output position.  A bin b* holding more than kCand codes
// (heavily tied rows) sends the row to the row path.  Same ordering and output
// as topk_row.  One size per power of two from 2048 to 32768 keys (4 to 64 a
// lane), so that no row pays for more than twice its own loads.
constexpr int kRowRegMin = 1024;     // shorter rows stay on the row path (cache-resident re-reads)
constexpr int kRowRegMax = 32768;

// Lanes below this one with their bit set in a wave mask.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                       __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u)));
}

template <int CAP>
__global__ __launch_bounds__(kTkThreads) void topk_row_reg_kernel(const float* __restrict__ keys,
                                                                  int n, int k, int n_sink,
                                                                  int n_local,
                                                                  int32_t* __restrict__ out,
                                                                  int stride) {
  constexpr int PER = CAP / kTkThreads;        // keys a lane
  constexpr int kWords = CAP / 64;             // bitmap words, one per (wave, e)
  constexpr int kBins = 4096;                  // first-pass histogram
  constexpr int kCand = 2048;                  // codes of the threshold bin kept for the exact pass
  static_assert(PER <= 64 && kWords <= kTkThreads, "one bitmap word per lane and per thread");
  __shared__ uint32_t s_bin[kBins];
  __shared__ uint32_t s_cand[kCand];
  __shared__ uint64_t s_gt[kWords];
  __shared__ uint64_t s_eq[kWords];
  __shared__ __align__(16) uint32_t hist[kKthHist];
  __shared__ int s_scan[2 * kTkWaves];
  __shared__ uint32_t s_red[2 * kTkWaves];
  __shared__ int s_wc[kTkWaves];
  __shared__ uint32_t s_bstar;
  __shared__ int s_need;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* o = out + size_t(row) * stride;
  const int lo = n_sink, hi = n - n_local, m = hi - lo;
  const int K = k < m ? k : m;
  write_fixed(o, n, n_sink, n_local, K, stride);
  if (K == m) {
    for (int i = tid; i < m; i += kTkThreads) o[n_sink + i] = lo + i;
    return;
  }
  if (K == 0) return;
  // 1. codes into registers
  const float* src = keys + size_t(row) * n + lo;
  const int wb = wave * 64 * PER + lane;       // this lane's first key
  uint32_t u[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) u[e] = f32_order_key(src[min(wb + 64 * e, m - 1)]);
  const int nfake = PER * kTkThreads - m;      // copies of the last key past the row end
  const uint32_t ulast = f32_order_key(src[m - 1]);
  uint32_t cmin = 0xFFFFFFFFu, cmax = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    cmin = u[e] < cmin ? u[e] : cmin;
    cmax = u[e] > cmax ? u[e] : cmax;
  }
  for (int i = tid; i < kBins; i += kTkThreads) s_bin[i] = 0;
  cmin = wave_minmax_u32<false>(cmin);
  cmax = wave_minmax_u32<true>(cmax);
  if (lane == 0) {
    s_red[wave] = cmin;
    s_red[kTkWaves + wave] = cmax;
  }
  __syncthreads();
  cmin = 0xFFFFFFFFu;
  cmax = 0u;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    cmin = s_red[w] < cmin ? s_red[w] : cmin;
    cmax = s_red[kTkWaves + w] > cmax ? s_red[kTkWaves + w] : cmax;
  }
  // 2. histogram of the codes in kBins bins of width 2^sh over [cmin, cmax],
  //    and the bin b* holding the K-th largest
  const int wbits = 32 - __clz(cmax - cmin);
  const int sh = wbits > 12 ? wbits - 12 : 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) atomicAdd(&s_bin[(u[e] - cmin) >> sh], 1u);
  if (tid == 0 && nfake) atomicSub(&s_bin[(ulast - cmin) >> sh], uint32_t(nfake));
  __syncthreads();
  {
    constexpr int BT = kBins / kTkThreads;            // bins BT*t .. BT*t+BT-1
    int cnt[BT], lsum = 0;
#pragma unroll
    for (int e = 0; e < BT; ++e) {
      cnt[e] = int(s_bin[BT * tid + e]);
      lsum += cnt[e];
    }
    int tot;
    const int before = block_scan1<false>(lsum, tot, s_scan);   // a barrier follows
    int above = tot - before - lsum;                  // codes in higher threads' bins
#pragma unroll
    for (int e = BT - 1; e >= 0; --e) {
      if (above < K && above + cnt[e] >= K) {
        s_bstar = uint32_t(BT * tid + e);
        s_need = K - above;
      }
      above += cnt[e];
    }
  }
  __syncthreads();
  const uint32_t bstar = s_bstar;
  int need = s_need;
  // 3. the codes of bin b* into a short list in index order (the copies of
  //    the last key, if they fall in b*, are its tail and are cut off)
  int c = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) c += __popcll(__ballot(((u[e] - cmin) >> sh) == bstar));
  if (lane == 0) s_wc[wave] = c;
  __syncthreads();
  int off = 0, ncand = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const int v = s_wc[w];
    off += w < wave ? v : 0;
    ncand += v;
  }
  if (ncand > kCand) {                                // a crowded bin: the row path
    topk_row<SDQ_KEY_F32_MAX>(keys, size_t(row) * n, n, k, n_sink, n_local, o, stride);
    return;
  }
  {
    const uint32_t blo = cmin + (bstar << sh);        // bin b* is [blo, blo + 2^sh)
    const uint32_t bw = sh >= 32 ? 0xFFFFFFFFu : (1u << sh);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool in = u[e] - blo < bw;
      const uint64_t mk = __ballot(in);
      if (in) s_cand[off + lanes_below(mk)] = u[e];
      off += __popcll(mk);
    }
  }
  if (((ulast - cmin) >> sh) == bstar) ncand -= nfake;
  __syncthreads();
  // 4. the exact K-th code and how many of its ties to keep (all codes above
  //    bin b* are in the top K already)
  const KthResult kr = select_kth(
      ncand, need,
      [&](int i, uint32_t* v) {
        *v = s_cand[i];
        return true;
      },
      hist, s_red);
  const uint32_t T = kr.T;
  need = kr.need;
  // 5. bitmaps of the codes above T and equal to T; lane e of the wave keeps
  //    the two ballots of its e-th keys
  uint32_t glo = 0, ghi = 0, qlo = 0, qhi = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const uint64_t gm = __ballot(u[e] > T);
    const uint64_t qm = __ballot(u[e] == T);
    if (lane == e) {
      glo = uint32_t(gm);
      ghi = uint32_t(gm >> 32);
      qlo = uint32_t(qm);
      qhi = uint32_t(qm >> 32);
    }
  }
  if (lane < PER) {
    s_gt[wave * PER + lane] = (uint64_t(ghi) << 32) | glo;
    s_eq[wave * PER + lane] = (uint64_t(qhi) << 32) | qlo;
  }
  __syncthreads();
  // thread t takes word t: keys 64 PER (t / PER) + 64 (t % PER) + [0, 64)
  const uint64_t gw = tid < kWords ? s_gt[tid] : 0ull;
  uint64_t qw = tid < kWords ? s_eq[tid] : 0ull;
  int gb, qb, gtot, qtot;
  block_scan2<false>(__popcll(gw), __popcll(qw), gb, qb, gtot, qtot, s_scan);
  int take = need - qb;                               // ties of this word that are kept
  take = take < 0 ? 0 : take;
  uint64_t qkeep = 0;
  for (int j = 0; j < take && qw; ++j) {
    const uint64_t b = qw & (~qw + 1);
    qkeep |= b;
    qw ^= b;
  }
  uint64_t bits = gw | qkeep;
  int pos = n_sink + gb + (qb < need ? qb : need);
  const int i0 = lo + (tid / PER) * 64 * PER + (tid % PER) * 64;
  const int end = n_sink + K;
  while (bits) {
    const int b = __ffsll((unsigned long long)bits) - 1;
    if (pos < end) o[pos] = i0 + b;
    ++pos;
    bits &= bits - 1;
  }
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
  // codes in bins of higher threads: the total minus this thread's inclusive
  // prefix (wave scans, then the four wave totals through LDS)
  const int inc = wave_incl_scan(tot);
  if ((tid & 63) == 63) s_part[tid >> 6] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < (tid >> 6) ? s_part[w] : 0;
    all += s_part[w];
  }
  int above = all - (before + inc);
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
  __shared__ __align__(16) uint32_t hist[kKthHist];
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
  __shared__ uint32_t s_red[2 * kTkWaves];
  const KthResult k2 = select_kth(
      cnt, K,
      [&](int i, uint32_t* u) {
        *u = uint32_t(ck[i] >> 32);
        return true;
      },
      hist, s_red);
  const KthResult k3 = select_kth(
      cnt, k2.need,
      [&](int i, uint32_t* u) {
        const uint64_t v = ck[i];
        *u = uint32_t(v);
        return uint32_t(v >> 32) == k2.T;
      },
      hist, s_red);
  const uint64_t prefix = (uint64_t(k2.T) << 32) | k3.T;   // exactly K composites are >= it
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


// ------------------------------------------------------------- uint8 path
// uint8 distances, smallest first.  One workgroup per row: a 256-bin
// histogram of the competition keys (wave-private LDS counters) gives the
// k-th smallest value T and how many of the keys equal to T to keep (the
// lowest-index ones); a block-wide prefix sum over the threads, whose keys
// are consecutive, places the winners in index order.  A thread holds 256
// keys (16-byte loads) per chunk of kU8Chunk keys; rows of one chunk are read
// once, longer rows twice.
constexpr int kU8PerThread = 256;
constexpr int kU8Chunk = kU8PerThread * kTkThreads;

// This thread's keys [s, s + cnt) of a chunk into w (bytes past cnt are 0).
__device__ __forceinline__ void u8_load(const uint8_t* rowp, int s, int cnt, uint4 (&w)[16]) {
  if (cnt == kU8PerThread && (reinterpret_cast<uintptr_t>(rowp + s) & 15) == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(rowp + s);
#pragma unroll
    for (int v = 0; v < 16; ++v) w[v] = p[v];
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      uint32_t d[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t x = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 16 * v + 4 * c + b;
          if (i < cnt) x |= uint32_t(rowp[s + i]) << (8 * b);
        }
        d[c] = x;
      }
      w[v] = make_uint4(d[0], d[1], d[2], d[3]);
    }
  }
}

__device__ __forceinline__ uint32_t u8_at(const uint4 (&w)[16], int i) {
  const uint4 v = w[i >> 4];
  const int c = (i >> 2) & 3;
  const uint32_t x = c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
  return (x >> (8 * (i & 3))) & 0xFFu;
}

__global__ __launch_bounds__(kTkThreads) void topk_u8_kernel(const uint8_t* __restrict__ keys, int n,
                                                             int k, int n_sink, int n_local,
                                                             int32_t* __restrict__ out, int stride) {
  __shared__ uint32_t hist[kTkWaves][256];
  __shared__ int s_scan[2 * kTkWaves];
  __shared__ int s_T, s_need;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* o = out + size_t(row) * stride;
  const int lo = n_sink, hi = n - n_local, m = hi - lo;
  const int K = k < m ? k : m;
  write_fixed(o, n, n_sink, n_local, K, stride);
  if (K == m) {
    for (int i = tid; i < m; i += kTkThreads) o[n_sink + i] = lo + i;
    return;
  }
  if (K == 0) return;
  const uint8_t* rowp = keys + size_t(row) * n;
  for (int i = tid; i < kTkWaves * 256; i += kTkThreads) (&hist[0][0])[i] = 0;
  __syncthreads();
  uint4 w[16];
  auto range = [&](int c0, int& s, int& cnt) {
    s = c0 + tid * kU8PerThread;
    const int e = s + kU8PerThread < hi ? s + kU8PerThread : hi;
    cnt = e > s ? e - s : 0;
  };
  // 1. histogram of the distances
  for (int c0 = lo; c0 < hi; c0 += kU8Chunk) {
    int s, cnt;
    range(c0, s, cnt);
    u8_load(rowp, s, cnt, w);
#pragma unroll
    for (int i = 0; i < kU8PerThread; ++i)                    // unrolled: w stays in registers
      if (i < cnt) atomicAdd(&hist[wave][u8_at(w, i)], 1u);
  }
  __syncthreads();
  // 2. T = the K-th smallest distance; need = how many of its ties to keep
  if (wave == 0) {
    int c[4], lsum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int t = 0;
#pragma unroll
      for (int wv = 0; wv < kTkWaves; ++wv) t += int(hist[wv][4 * lane + e]);
      c[e] = t;
      lsum += t;
    }
    const int inc = wave_incl_scan(lsum);
    int below = inc - lsum;                     // keys with distance < 4 * lane
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (below < K && below + c[e] >= K) {
        s_T = 4 * lane + e;
        s_need = K - below;
      }
      below += c[e];
    }
  }
  __syncthreads();
  const uint32_t T = uint32_t(s_T);
  const int need = s_need;
  // 3. winners in index order: d < T, and the first `need` keys with d == T
  int out_pos = n_sink, eq_seen = 0;
  const bool one_chunk = m <= kU8Chunk;
  for (int c0 = lo; c0 < hi; c0 += kU8Chunk) {
    int s, cnt;
    range(c0, s, cnt);
    if (!one_chunk) u8_load(rowp, s, cnt, w);
    // bit i of word i/32: key i of this thread has d < T (mlt) or d == T (meq)
    uint32_t mlt[kU8PerThread / 32], meq[kU8PerThread / 32];
#pragma unroll
    for (int v = 0; v < kU8PerThread / 32; ++v) {
      mlt[v] = 0;
      meq[v] = 0;
    }
#pragma unroll
    for (int i = 0; i < kU8PerThread; ++i) {
      const uint32_t d = u8_at(w, i);
      mlt[i / 32] |= uint32_t(i < cnt && d < T) << (i % 32);
      meq[i / 32] |= uint32_t(i < cnt && d == T) << (i % 32);
    }
    int lt = 0, eq = 0;
#pragma unroll
    for (int v = 0; v < kU8PerThread / 32; ++v) {
      lt += __popc(mlt[v]);
      eq += __popc(meq[v]);
    }
    int elt, eeq, tlt, teq;
    block_scan2(lt, eq, elt, eeq, tlt, teq, s_scan);
    const int eq_left = need - eq_seen > 0 ? need - eq_seen : 0;
    int pos = out_pos + elt + (eeq < eq_left ? eeq : eq_left);
    int allow = eq_left - eeq;                  // ties this thread may still take
    const int end = n_sink + K;
#pragma unroll
    for (int v = 0; v < kU8PerThread / 32; ++v) {
      uint32_t e = meq[v];
      for (; e && allow > 0; --allow) e &= e - 1;   // clear the first `allow` ties: kept
      uint32_t win = mlt[v] | (meq[v] & ~e);
      allow = allow > 0 ? allow : 0;
      for (; win; win &= win - 1) {
        if (pos < end) o[pos] = s + 32 * v + (__ffs(win) - 1);
        ++pos;
      }
    }
    out_pos += tlt + (teq < eq_left ? teq : eq_left);
    eq_seen += teq;
  }
}

// Many segments per row (long uint8 rows).  Pass 1: one workgroup per
// segment of kU8Seg keys writes the segment's 256-bin histogram to the
// workspace (LDS counters privatised per wave and lane quarter, so clustered
// distances do not serialise on one counter).  Pass 2: one workgroup per
// segment sums its row's histograms to find T and `need`, takes its place in
// the row from the histograms of the segments before it, and compacts its own
// winners in index order.  No counter is shared between workgroups.
constexpr int kU8SegThreads = 256;
constexpr int kU8SegPer = 64;                               // keys per thread
constexpr int kU8Seg = kU8SegThreads * kU8SegPer;           // 16384

__device__ __forceinline__ void u8_load64(const uint8_t* rowp, int s, int cnt, uint4 (&w)[4]) {
  if (cnt == kU8SegPer && (reinterpret_cast<uintptr_t>(rowp + s) & 15) == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(rowp + s);
#pragma unroll
    for (int v = 0; v < 4; ++v) w[v] = p[v];
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      uint32_t d[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t x = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 16 * v + 4 * c + b;
          if (i < cnt) x |= uint32_t(rowp[s + i]) << (8 * b);
        }
        d[c] = x;
      }
      w[v] = make_uint4(d[0], d[1], d[2], d[3]);
    }
  }
}

__device__ __forceinline__ uint32_t u8_at64(const uint4 (&w)[4], int i) {
  const uint4 v = w[i >> 4];
  const int c = (i >> 2) & 3;
  const uint32_t x = c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
  return (x >> (8 * (i & 3))) & 0xFFu;
}

__global__ __launch_bounds__(kU8SegThreads) void topk_u8_hist_kernel(const uint8_t* __restrict__ keys,
                                                                     int n, int lo, int hi, int nseg,
                                                                     uint32_t* __restrict__ ws) {
  constexpr int kCopies = (kU8SegThreads / 64) * 4;         // per wave and lane quarter
  __shared__ uint32_t h[kCopies][256];
  const int seg = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int copy = (tid >> 6) * 4 + (tid & 3);
  for (int i = tid; i < kCopies * 256; i += kU8SegThreads) (&h[0][0])[i] = 0;
  const int s = lo + seg * kU8Seg + tid * kU8SegPer;
  const int e = s + kU8SegPer < hi ? s + kU8SegPer : hi;
  const int cnt = e > s ? e - s : 0;
  uint4 w[4];
  u8_load64(keys + size_t(row) * n, s, cnt, w);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kU8SegPer; ++i)
    if (i < cnt) atomicAdd(&h[copy][u8_at64(w, i)], 1u);
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int c = 0; c < kCopies; ++c) t += h[c][tid];
  ws[(size_t(row) * nseg + seg) * 256 + tid] = t;
}

// Hamming distances and pass 1 in one launch (HashAttention study notes,
// sec. 2.1 SCORE then TOPK): one workgroup per segment of the competition
// range computes its tokens' distances popcount(sig XOR qsig), stores them,
// and writes the segment's 256-bin histogram in the layout
// topk_u8_hist_kernel writes.  A distance lies in [0, 32], so only 33 bins
// are counted (in LDS, privatised per wave and per lane sixteenth, odd row
// stride so that one bin's copies fall in different banks: a bin's LDS
// atomics meet at most 4 lanes of a wave) and the rest are zero.
// 1024 threads of 16 tokens cover one segment.  One more workgroup per row
// stores the distances of the sink and local windows [0, lo) and [hi, n).
// Signature rows are n_cap long.
constexpr int kHhThreads = 1024;
constexpr int kHhPer = kU8Seg / kHhThreads;                // 16 tokens per thread
constexpr int kHhBins = 33;
constexpr int kHhWaves = kHhThreads / 64;
constexpr int kHhCopies = 16;                              // histogram copies per wave

__global__ __launch_bounds__(kHhThreads) void hamming_hist_kernel(
    const uint32_t* __restrict__ sigs, const uint32_t* __restrict__ qsig, int n, int n_cap, int lo,
    int hi, int nseg, uint8_t* __restrict__ dist, uint32_t* __restrict__ ws) {
  __shared__ uint32_t h[kHhWaves * kHhCopies][kHhBins];
  const int seg = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const uint32_t qs = qsig[row];
  const uint32_t* srow = sigs + size_t(row) * n_cap;
  uint8_t* drow = dist + size_t(row) * n;
  if (seg == nseg) {
    for (int i = tid; i < lo; i += kHhThreads) drow[i] = uint8_t(__popc(srow[i] ^ qs));
    for (int i = hi + tid; i < n; i += kHhThreads) drow[i] = uint8_t(__popc(srow[i] ^ qs));
    return;
  }
  const int copy = (tid >> 6) * kHhCopies + (tid & (kHhCopies - 1));
  for (int i = tid; i < kHhWaves * kHhCopies * kHhBins; i += kHhThreads) (&h[0][0])[i] = 0;
  const int s = lo + seg * kU8Seg + tid * kHhPer;
  const int e = s + kHhPer < hi ? s + kHhPer : hi;
  const int cnt = e > s ? e - s : 0;
  uint32_t dw[kHhPer / 4];                                   // 4 distances per word
  if (cnt == kHhPer && (reinterpret_cast<uintptr_t>(srow + s) & 15) == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(srow + s);
    uint4 v[kHhPer / 4];
#pragma unroll
    for (int j = 0; j < kHhPer / 4; ++j) v[j] = p[j];
#pragma unroll
    for (int j = 0; j < kHhPer / 4; ++j)
      dw[j] = uint32_t(__popc(v[j].x ^ qs)) | (uint32_t(__popc(v[j].y ^ qs)) << 8) |
              (uint32_t(__popc(v[j].z ^ qs)) << 16) | (uint32_t(__popc(v[j].w ^ qs)) << 24);
  } else {
#pragma unroll
    for (int j = 0; j < kHhPer / 4; ++j) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i = 4 * j + b;
        if (i < cnt) x |= uint32_t(__popc(srow[s + i] ^ qs)) << (8 * b);
      }
      dw[j] = x;
    }
  }
  if (cnt == kHhPer && (reinterpret_cast<uintptr_t>(drow + s) & 15) == 0) {
    *reinterpret_cast<uint4*>(drow + s) = make_uint4(dw[0], dw[1], dw[2], dw[3]);
  } else {
#pragma unroll
    for (int i = 0; i < kHhPer; ++i)
      if (i < cnt) drow[s + i] = uint8_t((dw[i >> 2] >> (8 * (i & 3))) & 0xFFu);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kHhPer; ++i)
    if (i < cnt) atomicAdd(&h[copy][(dw[i >> 2] >> (8 * (i & 3))) & 0xFFu], 1u);
  __syncthreads();
  // each wave's copies into its first, then the waves' sums per bin
  if (tid < kHhWaves * kHhBins) {
    const int w = tid / kHhBins, bin = tid - w * kHhBins;
    uint32_t t = 0;
#pragma unroll
    for (int c = 0; c < kHhCopies; ++c) t += h[kHhCopies * w + c][bin];
    h[kHhCopies * w][bin] = t;
  }
  __syncthreads();
  if (tid < 256) {
    uint32_t t = 0;
    if (tid < kHhBins) {
#pragma unroll
      for (int w = 0; w < kHhWaves; ++w) t += h[kHhCopies * w][tid];
    }
    ws[(size_t(row) * nseg + seg) * 256 + tid] = t;
  }
}

__global__ __launch_bounds__(kU8SegThreads) void topk_u8_select_kernel(
    const uint8_t* __restrict__ keys, int n, int k, int n_sink, int n_local, int nseg,
    const uint32_t* __restrict__ ws, int32_t* __restrict__ out, int stride) {
  __shared__ int s_red[2 * (kU8SegThreads / 64)];
  __shared__ int s_T, s_need;
  const int seg = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int W = kU8SegThreads / 64;
  int32_t* o = out + size_t(row) * stride;
  const int lo = n_sink, hi = n - n_local, m = hi - lo;
  const int K = k < m ? k : m;                               // 0 < K < m here
  if (seg == 0) write_fixed(o, n, n_sink, n_local, K, stride);
  // thread d: distance d's count over the row and over the segments before this one
  const uint32_t* hr = ws + size_t(row) * nseg * 256;
  // eight loads in flight per batch (clamped indices keep them unconditional)
  int tot = 0, before = 0;
  for (int s0 = 0; s0 < nseg; s0 += 8) {
    uint32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sg = s0 + u < nseg ? s0 + u : nseg - 1;
      c[u] = hr[size_t(sg) * 256 + tid];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = s0 + u < nseg ? int(c[u]) : 0;
      tot += v;
      if (s0 + u < seg) before += v;
    }
  }
  // T: smallest d with (count of keys <= d) >= K; prefix over d = tid
  int inc = wave_incl_scan(tot);
  if (lane == 63) s_red[wave] = inc;
  __syncthreads();
  int wbase = 0;
#pragma unroll
  for (int w = 0; w < W; ++w)
    if (w < wave) wbase += s_red[w];
  inc += wbase;                                              // keys with distance <= tid
  if (inc >= K && inc - tot < K) {
    s_T = tid;
    s_need = K - (inc - tot);
  }
  __syncthreads();
  const int T = s_T, need = s_need;
  // keys of earlier segments with d < T, and with d == T
  int blt = tid < T ? before : 0;
  const int beq = (tid == T) ? before : 0;
  __syncthreads();
  blt = wave_sum_dpp(blt);
  const int beq_w = wave_sum_dpp(beq);
  if (lane == 0) {
    s_red[wave] = blt;
    s_red[W + wave] = beq_w;
  }
  __syncthreads();
  int lt_before = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    lt_before += s_red[w];
    eq_before += s_red[W + w];
  }
  __syncthreads();
  // this segment's keys: winners in index order
  const int s = lo + seg * kU8Seg + tid * kU8SegPer;
  const int e = s + kU8SegPer < hi ? s + kU8SegPer : hi;
  const int cnt = e > s ? e - s : 0;
  uint4 w4[4];
  u8_load64(keys + size_t(row) * n, s, cnt, w4);
  uint32_t mlt[2] = {0u, 0u}, meq[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < kU8SegPer; ++i) {
    const uint32_t d = u8_at64(w4, i);
    mlt[i / 32] |= uint32_t(i < cnt && int(d) < T) << (i % 32);
    meq[i / 32] |= uint32_t(i < cnt && int(d) == T) << (i % 32);
  }
  const int lt = __popc(mlt[0]) + __popc(mlt[1]);
  const int eq = __popc(meq[0]) + __popc(meq[1]);
  int elt, eeq, tlt, teq;
  {
    // exclusive prefix over the workgroup of (lt, eq)
    const int ia = wave_incl_scan(lt), ib = wave_incl_scan(eq);
    if (lane == 63) {
      s_red[wave] = ia;
      s_red[W + wave] = ib;
    }
    __syncthreads();
    int wa = 0, wb = 0;
    tlt = 0;
    teq = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      if (w < wave) {
        wa += s_red[w];
        wb += s_red[W + w];
      }
      tlt += s_red[w];
      teq += s_red[W + w];
    }
    elt = wa + ia - lt;
    eeq = wb + ib - eq;
  }
  (void)tlt;
  (void)teq;
  const int eq_left = need - eq_before > 0 ? need - eq_before : 0;
  const int eq_taken_before = eq_before < need ? eq_before : need;
  int pos = n_sink + lt_before + eq_taken_before + elt + (eeq < eq_left ? eeq : eq_left);
  int allow = eq_left - eeq;
  const int end = n_sink + K;
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    uint32_t ee = meq[v];
    for (; ee && allow > 0; --allow) ee &= ee - 1;           // the first `allow` ties are kept
    uint32_t win = mlt[v] | (meq[v] & ~ee);
    allow = allow > 0 ? allow : 0;
    for (; win; win &= win - 1) {
      if (pos < end) o[pos] = s + 32 * v + (__ffs(win) - 1);
      ++pos;
    }
  }
}

// ------------------------------------------------------------- block-max path
// Rows whose competition range is made of whole 64-key blocks.  With M_b the
// maximum of block b, the k-th largest block maximum T satisfies T <= the
// k-th largest key (the k blocks whose maxima are >= T hold k keys >= T), so
// every key of the exact top-k lies in a block with M_b >= T and is >= T.
// One workgroup per row, no sorting:
//  1. thread t holds the maxima of competition blocks [32t, 32t+32) in
//     registers;
//  2. a 4096-bin histogram of their order-preserving codes over the row's
//     [min, max] code range locates the bin b* holding the k-th largest
//     maximum; its lower edge is a float threshold thr <= T, so the top-k
//     keys are among the keys >= thr;
//  3. candidate blocks (M_b >= thr) are listed in index order (one prefix
//     sum over the threads, whose blocks are consecutive);
//  4. thread t takes candidate blocks t, t + 512, ... (whole blocks: 256 B
//     from each lane), counts its keys >= thr, and one prefix sum places
//     them in index order;
//  5. the exact k-th largest candidate code and its tie count are found;
//  6. the winners are written by an index-ordered compaction (ties to the
//     lower index), so the output comes out ascending.
// The workgroup's steps are dependent latencies (a load, an LDS round trip,
// a barrier), so each step is one pass of straight-line per-thread work.
// Rows whose candidates overflow the lists fall back to the row path.  Keys
// must not be NaN.
constexpr int kBmMaxBlocks = 16384;     // n <= 2^20
constexpr int kBmPer = kBmMaxBlocks / kTkThreads;   // block maxima per thread
constexpr int kBmBins = 4096;
constexpr int kBmCandBlocks = 2048;     // candidate blocks (at most 4 per thread)
constexpr int kBmCap = 2048;            // candidate keys

__global__ __launch_bounds__(256) void topk_block_max_kernel(const float* __restrict__ keys, int n,
                                                             int nb, float* __restrict__ bm) {
  const int row = blockIdx.y;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= nb) return;
  float v = keys[size_t(row) * n + size_t(b) * 64 + (threadIdx.x & 63)];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  if ((threadIdx.x & 63) == 0) bm[size_t(row) * nb + b] = v;
}

// Inverse of f32_order_key on the codes of non-NaN floats (+0 for the code
// of zero).
__device__ __forceinline__ float f32_from_order_key(uint32_t c) {
  return __uint_as_float((c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c);
}


// Candidate keys kept as floats (converted to order codes when read: cheaper
// in the collection loop) or as order codes (the split form's workspace).
__device__ __forceinline__ uint32_t ckey_code(uint32_t c) { return c; }
__device__ __forceinline__ uint32_t ckey_code(float v) { return f32_order_key(v); }
// The lower edge (an order code) of the kBmBins-bin histogram bin, over the
// code range [cmin, cmax], that holds the K-th largest of the values v[u]
// whose bit u of `in` is set (all threads of the workgroup call it; sbin
// cleared before a barrier that precedes the call).  At least K values must
// be counted; otherwise the result is cmin.
template <int PER>
__device__ __forceinline__ uint32_t bm_kth_bin_edge(const float (&v)[PER], uint32_t in, int K,
                                                    uint32_t cmin, uint32_t cmax, uint32_t* sbin,
                                                    int* s_scan, uint32_t* s_thr) {
  const int tid = threadIdx.x;
  // bins of width 2^sh over [cmin, cmax]: (cmax - cmin) >> sh < kBmBins
  const int wbits = 32 - __clz(cmax - cmin);
  const int sh = wbits > 12 ? wbits - 12 : 0;
  if (tid == 0) *s_thr = cmin;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if ((in >> u) & 1u) atomicAdd(&sbin[(f32_order_key(v[u]) - cmin) >> sh], 1u);
  __syncthreads();
  {
    constexpr int BT = kBmBins / kTkThreads;           // bins BT*t .. BT*t+BT-1
    int cnt[BT], lsum = 0;
#pragma unroll
    for (int e = 0; e < BT; ++e) {
      cnt[e] = sbin[BT * tid + e];
      lsum += cnt[e];
    }
    int tot;
    const int before = block_scan1<false>(lsum, tot, s_scan);   // a barrier follows
    int above = tot - before - lsum;                     // values in higher threads' bins
#pragma unroll
    for (int e = BT - 1; e >= 0; --e) {
      if (above < K && above + cnt[e] >= K) (*s_thr) = cmin + (uint32_t(BT * tid + e) << sh);
      above += cnt[e];
    }
  }
  __syncthreads();
  return *s_thr;
}

// Phases 1-3 of the block-max path for one row (all threads of the
// workgroup call it): the threshold thr <= the K-th largest key from the
// row's block maxima brow[0..nbc), and the blocks whose maximum reaches it,
// in index order, in cb[0..ncb); cmax_out is the order code of the row's
// largest key (its largest block maximum).  Returns false (cb not written) when more
// than kBmCandBlocks blocks qualify.
__device__ __forceinline__ bool bm_candidate_blocks(const float* __restrict__ brow, int nbc, int K,
                                                    uint32_t* sbin, int* cb, uint32_t* s_red,
                                                    int* s_scan, uint32_t* s_thr, float& thr_out,
                                                    int& ncb_out, uint32_t& cmax_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // 1. this thread's block maxima (blocks past the end read as -inf)
  const int b0 = tid * kBmPer;
  float mx[kBmPer];
  if ((reinterpret_cast<uintptr_t>(brow) & 15) == 0 && b0 + kBmPer <= nbc) {
#pragma unroll
    for (int u = 0; u < kBmPer; u += 4) {
      const float4 v = *reinterpret_cast<const float4*>(brow + b0 + u);
      mx[u] = v.x;
      mx[u + 1] = v.y;
      mx[u + 2] = v.z;
      mx[u + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < kBmPer; ++u) mx[u] = b0 + u < nbc ? brow[b0 + u] : -INFINITY;
  }
  for (int i = tid; i < kBmBins; i += kTkThreads) sbin[i] = 0;
  // code range of the maxima
  uint32_t cmin = 0xFFFFFFFFu, cmax = 0u;
#pragma unroll
  for (int u = 0; u < kBmPer; ++u) {
    if (b0 + u < nbc) {
      const uint32_t cd = f32_order_key(mx[u]);
      cmin = cd < cmin ? cd : cmin;
      cmax = cd > cmax ? cd : cmax;
    }
  }
  cmin = wave_minmax_u32<false>(cmin);
  cmax = wave_minmax_u32<true>(cmax);
  if (lane == 0) {
    s_red[wave] = cmin;
    s_red[kTkWaves + wave] = cmax;
  }
  __syncthreads();
  cmin = 0xFFFFFFFFu;
  cmax = 0u;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    cmin = s_red[w] < cmin ? s_red[w] : cmin;
    cmax = s_red[kTkWaves + w] > cmax ? s_red[kTkWaves + w] : cmax;
  }
  cmax_out = cmax;                                     // the row's largest key
  // bins of width 2^sh over [cmin, cmax]: (cmax - cmin) >> sh < kBmBins
  const int wbits = 32 - __clz(cmax - cmin);
  const int sh = wbits > 12 ? wbits - 12 : 0;
  // 2. histogram; bin b* holding the K-th largest maximum (the search of
  //    bm_kth_bin_edge, written out here: called with 32 values a thread the
  //    compiler scheduled the whole kernel 0.5 us slower)
#pragma unroll
  for (int u = 0; u < kBmPer; ++u)
    if (b0 + u < nbc) atomicAdd(&sbin[(f32_order_key(mx[u]) - cmin) >> sh], 1u);
  __syncthreads();
  {
    constexpr int BT = kBmBins / kTkThreads;           // bins BT*t .. BT*t+BT-1
    int cnt[BT], lsum = 0;
#pragma unroll
    for (int e = 0; e < BT; ++e) {
      cnt[e] = sbin[BT * tid + e];
      lsum += cnt[e];
    }
    int tot;
    const int before = block_scan1<false>(lsum, tot, s_scan);   // a barrier follows
    int above = tot - before - lsum;                     // maxima in higher threads' bins
#pragma unroll
    for (int e = BT - 1; e >= 0; --e) {
      if (above < K && above + cnt[e] >= K) (*s_thr) = cmin + (uint32_t(BT * tid + e) << sh);
      above += cnt[e];
    }
  }
  __syncthreads();
  const float thr = f32_from_order_key(*s_thr);          // v >= thr  <=>  bin(v) >= b*
  thr_out = thr;
  // 3. candidate blocks in index order
  uint32_t flags = 0;
#pragma unroll
  for (int u = 0; u < kBmPer; ++u) flags |= uint32_t(mx[u] >= thr) << u;   // -inf never passes
  int ncb;
  const int cpos = block_scan1<false>(__popc(flags), ncb, s_scan);   // a barrier follows
  ncb_out = ncb;
  if (ncb > kBmCandBlocks) return false;
  {
    int pos = cpos;
    for (uint32_t f = flags; f; f &= f - 1) cb[pos++] = b0 + __ffs(f) - 1;
  }
  __syncthreads();
  return true;
}

// Phase 4: the keys >= thr of the candidate blocks cb[0..ncb) (block
// numbers from blo), in index order, into ckey and their indices into cidx
// (both of `cap` entries).  Returns their count; when it exceeds
// cap nothing more is written (the caller then falls back).  kRC rounds of
// 32 blocks are in flight at once; s_cnt holds 32 kRC entries.
template <int kRC>
__device__ __forceinline__ int bm_collect(const float* __restrict__ keys, size_t base, int blo,
                                          const int* cb, int ncb, float thr, float* ckey, int* cidx,
                                          int cap, int* s_cnt,
                          int* s_scan) {
  const int tid = threadIdx.x;
  // 4. candidate keys in index order.  16 lanes share a block (lane q holds
  //    its keys 4q..4q+3), so a wave load covers four whole blocks; a chunk
  //    of kRC rounds x 32 blocks is in flight at once.  Per-lane counts of
  //    keys >= thr travel four rounds to an int in 8-bit fields through the
  //    in-group sums and prefixes; a prefix sum over the chunk's blocks
  //    places them.
  constexpr int kPk = kRC / 4;                          // packed counters
  const int grp = tid >> 4, q = tid & 15;
  int nc = 0;
  for (int cc = 0; cc < ncb; cc += kRC * 32) {
    const int nch = ncb - cc < kRC * 32 ? ncb - cc : kRC * 32;
    float4 v[kRC];
#pragma unroll
    for (int r = 0; r < kRC; ++r) {
      const int c = r * 32 + grp;                       // block within the chunk
      const int cl = cc + (c < nch ? c : nch - 1);      // clamped: loads stay unconditional
      v[r] = *reinterpret_cast<const float4*>(keys + base + size_t(blo + cb[cl]) * 64 + 4 * q);
    }
    uint32_t pk[kPk];
#pragma unroll
    for (int e = 0; e < kPk; ++e) pk[e] = 0;
#pragma unroll
    for (int r = 0; r < kRC; ++r) {
      const uint32_t k4 = uint32_t(v[r].x >= thr) + uint32_t(v[r].y >= thr) +
                          uint32_t(v[r].z >= thr) + uint32_t(v[r].w >= thr);
      pk[r / 4] |= k4 << (8 * (r % 4));
    }
    // inclusive prefix over the 16 lanes of the group (fields never exceed 64)
    uint32_t inc[kPk];
#pragma unroll
    for (int e = 0; e < kPk; ++e) {
      inc[e] = uint32_t(row16_incl_scan(int(pk[e])));
    }
    if (q == 15) {
#pragma unroll
      for (int r = 0; r < kRC; ++r) {
        const int c = r * 32 + grp;
        if (c < nch) s_cnt[c] = int((inc[r / 4] >> (8 * (r % 4))) & 0xFFu);
      }
    }
    __syncthreads();
    {
      constexpr int PT = (kRC * 32 + kTkThreads - 1) / kTkThreads;
      int cnt[PT], sum = 0;
#pragma unroll
      for (int e = 0; e < PT; ++e) {
        const int i = tid * PT + e;
        cnt[e] = i < nch ? s_cnt[i] : 0;
        sum += cnt[e];
      }
      int tot;
      int off = nc + block_scan1<false>(sum, tot, s_scan);           // a barrier follows
#pragma unroll
      for (int e = 0; e < PT; ++e) {
        const int i = tid * PT + e;
        if (i < nch) s_cnt[i] = off;
        off += cnt[e];
      }
      nc += tot;
    }
    __syncthreads();
    if (nc <= cap) {
      int offs[kRC], firsts[kRC];                       // every LDS read issued up front
#pragma unroll
      for (int r = 0; r < kRC; ++r) {
        const int c = r * 32 + grp;
        offs[r] = s_cnt[c < nch ? c : nch - 1];
        firsts[r] = (blo + cb[cc + (c < nch ? c : 0)]) * 64 + 4 * q;
      }
      // candidates are sparse (about one per block): a round is skipped
      // unless some lane of the wave holds one, and inside a round only the
      // kept keys are written (under the lane mask)
#pragma unroll
      for (int r = 0; r < kRC; ++r) {
        const int c = r * 32 + grp;
        const uint32_t mine = c < nch ? (pk[r / 4] >> (8 * (r % 4))) & 0xFFu : 0u;
        if (__ballot(mine != 0) == 0) continue;         // wave-uniform
        const uint32_t before = ((inc[r / 4] >> (8 * (r % 4))) & 0xFFu) - mine;
        int pos = offs[r] + int(before);
        const int first = firsts[r];
        const float xs[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = c < nch && xs[e] >= thr;
          if (keep) {
            ckey[pos] = xs[e];
            cidx[pos] = first + e;
          }
          pos += keep;
        }
      }
    }
    __syncthreads();
  }
  return nc;
}

// Phase 6: the winners in index order (candidates are already ordered by
// index): every key above kr.T and the first kr.need equal to it, after the
// fixed windows.
template <typename CK>
__device__ __forceinline__ void bm_write_winners(const CK* ckey, const int* cidx, int nc, int K,
                                                 KthResult kr, int n, int n_sink, int n_local,
                                                 int stride, int32_t* __restrict__ o,
                                                 int* s_scan) {
  const int tid = threadIdx.x;
  // 6. winners in index order (candidates are already ordered by index)
  write_fixed(o, n, n_sink, n_local, K, stride);
  int out_pos = n_sink, eq_seen = 0;
  constexpr int IPT = 4;
  for (int c0 = 0; c0 < nc; c0 += kTkThreads * IPT) {
    const int i0 = c0 + tid * IPT;
    uint32_t u[IPT];
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      const int i = i0 + e;
      u[e] = i < nc ? ckey_code(ckey[i]) : 0u;
      if (i < nc) {
        gt += u[e] > kr.T;
        eq += u[e] == kr.T;
      }
    }
    int egt, eeq, tgt, teq;
    block_scan2<false>(gt, eq, egt, eeq, tgt, teq,
                       s_scan + 2 * kTkWaves * ((c0 / (kTkThreads * IPT)) & 1));
    const int eq_left = kr.need - eq_seen > 0 ? kr.need - eq_seen : 0;
    int pos = out_pos + egt + (eeq < eq_left ? eeq : eq_left);
    int my_eq = eeq;
    const int end = n_sink + K;
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      const int i = i0 + e;
      if (i < nc) {
        if (u[e] > kr.T) {
          if (pos < end) o[pos] = cidx[i];
          ++pos;
        } else if (u[e] == kr.T) {
          if (my_eq < eq_left) {
            if (pos < end) o[pos] = cidx[i];
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

// Phases 5-6: the exact K-th largest of the candidate keys ckey[0..nc) and
// its tie count, then the winners.
template <typename CK>
__device__ __forceinline__ void bm_select_write(const CK* ckey, const int* cidx, int nc, int K,
                                                int n, int n_sink, int n_local, int stride,
                                                int32_t* __restrict__ o, uint32_t* hist,
                                                uint32_t* s_red, int* s_scan) {
  const KthResult kr = select_kth(
      nc, K,
      [&](int i, uint32_t* u) {
        *u = ckey_code(ckey[i]);
        return true;
      },
      hist, s_red);
  bm_write_winners(ckey, cidx, nc, K, kr, n, n_sink, n_local, stride, o, s_scan);
}

__global__ __launch_bounds__(kTkThreads) void topk_bm_kernel(const float* __restrict__ keys,
                                                             const float* __restrict__ bm, int n,
                                                             int nb, int k, int n_sink, int n_local,
                                                             int32_t* __restrict__ out, int stride) {
  __shared__ __align__(16) uint32_t sbin[kBmBins];
  __shared__ int cb[kBmCandBlocks];       // candidate block numbers, ascending
  __shared__ int s_cnt[640];              // kept keys per block of a chunk, then offsets
  __shared__ float ckey[kBmCap];
  __shared__ int cidx[kBmCap];
  __shared__ __align__(16) uint32_t hist[kKthHist];
  __shared__ uint32_t s_red[2 * kTkWaves];
  __shared__ int s_scan[4 * kTkWaves];    // two buffers: scans alternate
  __shared__ uint32_t s_thr;
  const int row = blockIdx.x;
  int32_t* o = out + size_t(row) * stride;
  const int lo = n_sink, hi = n - n_local, m = hi - lo;
  const int blo = lo / 64, nbc = m / 64;        // competition blocks [blo, blo + nbc)
  const int K = k < m ? k : m;
  const size_t base = size_t(row) * n;
  if (K == m || K == 0 || K > nbc) {
    topk_row<SDQ_KEY_F32_MAX>(keys, base, n, k, n_sink, n_local, o, stride);
    return;
  }
  float thr;
  int ncb;
  uint32_t cmax;
  if (!bm_candidate_blocks(bm + size_t(row) * nb + blo, nbc, K, sbin, cb, s_red, s_scan, &s_thr,
                           thr, ncb, cmax)) {
    topk_row<SDQ_KEY_F32_MAX>(keys, base, n, k, n_sink, n_local, o, stride);
    return;
  }
  const int nc = bm_collect<20>(keys, base, blo, cb, ncb, thr, ckey, cidx, kBmCap, s_cnt, s_scan);
  if (nc > kBmCap || nc < K) {
    topk_row<SDQ_KEY_F32_MAX>(keys, base, n, k, n_sink, n_local, o, stride);
    return;
  }
  bm_select_write(ckey, cidx, nc, K, n, n_sink, n_local, stride, o, hist, s_red, s_scan);
}

// Split form (topk_select_block_max_split): kBmSegs workgroups per row each
// derive the same threshold, collect the candidate keys of their own share of
// the row and leave them, in index order, in the workspace; one workgroup per
// row then selects exactly among all of them and writes the winners.  The
// candidate gather, one CU's load per row in the single-workgroup form, is
// spread over kBmSegs CUs.  With group maxima the threshold comes from those
// (one value per kBmGrp blocks) and each workgroup lists the candidate blocks
// of a contiguous eighth of the row from that eighth's block maxima, so no
// workgroup reads all of the row's block maxima; without them (or with fewer
// than K whole groups) every workgroup derives the threshold and the full
// candidate block list from all block maxima (phases 1-3) and takes a
// contiguous share of the list.  Any threshold <= the K-th largest key is
// exact here: the final selection is exact over whatever the segments keep.
// Each segment also leaves a 256-bin histogram of its candidates' code
// offsets above code(thr), a base every segment knows (bins finer near it,
// bm_seg_bin), so the final kernel starts its exact search inside the bin of
// the K-th key, cut at the code of the row's largest key.
// Workspace per row: a 64-byte header (the segments' counts, then the two
// range codes), the segments' codes, their indices, their histograms.
constexpr int kBmSegs = 8;
constexpr int kBmSegCap = kBmCap;       // candidate keys per segment
constexpr int kBmSegBins = 256;
constexpr int kBmGrp = SDQ_GROUP_BLOCKS;          // blocks per group maximum
constexpr int kBmGrpPer = kBmMaxBlocks / kBmGrp / kTkThreads;   // group maxima per thread
constexpr int kBmSegPer = kBmMaxBlocks / kBmSegs / kTkThreads;  // a segment's blocks per thread
static_assert(kBmGrpPer == 4 && kBmSegPer == 4, "one round of loads per thread");

__host__ __device__ inline size_t bm_split_ws_per_row() {
  return 64 + size_t(kBmSegs) * (kBmSegCap * 8 + kBmSegBins * 4);
}

// Segment histogram bins over the offset d = code - code(thr), finer near
// the threshold, where the K-th key lies (most candidates sit just above
// it): offsets below 8 take a bin each, and above that every octave
// [2^e, 2^(e+1)) splits into 8 bins of width 2^(e-3).  Bin order is offset
// order; bins 0..239 cover every 32-bit offset.
__device__ __forceinline__ uint32_t bm_seg_bin(uint32_t d) {
  const int e = 31 - __clz(d | 8u);                    // 3..31
  const uint32_t b = uint32_t(8 * (e - 2)) + ((d >> (e - 3)) & 7u);
  return d < 8 ? d : b;
}

// first offset of bin b, and its width less one
__device__ __forceinline__ void bm_seg_bin_range(uint32_t b, uint32_t& off, uint32_t& span) {
  const int s = int(b >> 3) - 1;                        // e - 3
  off = b < 8 ? b : (8u + (b & 7u)) << s;
  span = b < 8 ? 0u : (1u << s) - 1u;
}
static_assert(8 * 29 + 7 < kBmSegBins, "offset bins fit the segment histogram");

// v = p[i0 .. i0 + 4), entries at or past `end` read as -inf: one 16-byte load
// when all four are in range and p + i0 is 16-byte aligned (single loads
// with a 16-byte stride between lanes would pass four times the addresses
// through the CU's address unit).
__device__ __forceinline__ void load4_or_neg_inf(const float* __restrict__ p, int i0, int end,
                                                 float (&v)[4]) {
  if (i0 + 4 <= end && (reinterpret_cast<uintptr_t>(p + i0) & 15) == 0) {
    const float4 x = *reinterpret_cast<const float4*>(p + i0);
    v[0] = x.x;
    v[1] = x.y;
    v[2] = x.z;
    v[3] = x.w;
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i0 + u < end ? p[i0 + u] : -INFINITY;
  }
}

// Threshold from the group maxima (all threads of the workgroup call it).
// Groups [gi0, gi1) lie wholly inside the competition blocks: the K-th
// largest of their maxima, T', is <= the K-th largest block maximum T (the K
// groups whose maxima are >= T' each hold a competition block whose maximum
// is their group's), so thr = the lower edge of the histogram bin holding T'
// is a valid threshold, and it reads 16 times fewer values than T does.
// Groups [gc0, gc1) meet the competition blocks: their largest maximum
// bounds every competing key (cmax_out).  gi1 - gi0 >= K.
__device__ __forceinline__ float bm_group_threshold(const float* __restrict__ grow, int gi0, int gi1,
                                                    int gc0, int gc1, int K, uint32_t* sbin,
                                                    uint32_t* s_red, int* s_scan, uint32_t* s_thr,
                                                    uint32_t& cmax_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g0 = gc0 + tid * kBmGrpPer;
  float gv[kBmGrpPer];
  load4_or_neg_inf(grow, g0, gc1, gv);
  for (int i = tid; i < kBmBins; i += kTkThreads) sbin[i] = 0;
  uint32_t in = 0, cmin = 0xFFFFFFFFu, cimax = 0u, cmax = 0u;
#pragma unroll
  for (int u = 0; u < kBmGrpPer; ++u) {
    const int gi = g0 + u;
    const uint32_t cd = f32_order_key(gv[u]);
    if (gi < gc1) cmax = cd > cmax ? cd : cmax;
    if (gi >= gi0 && gi < gi1) {
      in |= 1u << u;
      cmin = cd < cmin ? cd : cmin;
      cimax = cd > cimax ? cd : cimax;
    }
  }
  cmin = wave_minmax_u32<false>(cmin);
  cimax = wave_minmax_u32<true>(cimax);
  cmax = wave_minmax_u32<true>(cmax);
  if (lane == 0) {
    s_red[wave] = cmin;
    s_red[kTkWaves + wave] = cimax;
    s_red[2 * kTkWaves + wave] = cmax;
  }
  __syncthreads();
  cmin = 0xFFFFFFFFu;
  cimax = 0u;
  cmax = 0u;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    cmin = s_red[w] < cmin ? s_red[w] : cmin;
    cimax = s_red[kTkWaves + w] > cimax ? s_red[kTkWaves + w] : cimax;
    cmax = s_red[2 * kTkWaves + w] > cmax ? s_red[2 * kTkWaves + w] : cmax;
  }
  cmax_out = cmax;
  return f32_from_order_key(bm_kth_bin_edge(gv, in, K, cmin, cimax, sbin, s_scan, s_thr));
}

// The blocks [sb0, sb1) of brow (at most kTkThreads * kBmSegPer) whose
// maximum reaches thr, in index order, into cb; returns their count.  bv
// holds this thread's maxima, blocks sb0 + kBmSegPer * tid + u.
__device__ __forceinline__ int bm_list_blocks(const float (&bv)[kBmSegPer], int sb0, int sb1,
                                              float thr, int* cb, int* s_scan) {
  const int tid = threadIdx.x;
  const int b0 = sb0 + tid * kBmSegPer;
  uint32_t flags = 0;
#pragma unroll
  for (int u = 0; u < kBmSegPer; ++u) flags |= uint32_t(b0 + u < sb1 && bv[u] >= thr) << u;
  int ncb;
  int pos = block_scan1<false>(__popc(flags), ncb, s_scan);   // a barrier follows
  for (uint32_t f = flags; f; f &= f - 1) cb[pos++] = b0 + __ffs(f) - 1;
  __syncthreads();
  return ncb;
}

// GROUPS: the threshold from the group maxima gm (the host has checked
// that at least K groups lie wholly inside the competition blocks), else
// from all block maxima.
template <bool GROUPS>
__global__ __launch_bounds__(kTkThreads) void topk_bm_seg_kernel(const float* __restrict__ keys,
                                                                 const float* __restrict__ bm,
                                                                 const float* __restrict__ gm,
                                                                 int n, int nb, int k, int n_sink,
                                                                 int n_local, void* ws) {
  __shared__ __align__(16) uint32_t sbin[kBmBins];
  __shared__ int cb[kBmCandBlocks];
  __shared__ int s_cnt[128];
  __shared__ float ckey[kBmSegCap];
  __shared__ int cidx[kBmSegCap];
  __shared__ uint32_t s_red[(GROUPS ? 3 : 2) * kTkWaves];
  __shared__ int s_scan[4 * kTkWaves];
  __shared__ uint32_t s_thr;
  __shared__ uint32_t s_h[kBmSegBins];
  const int seg = blockIdx.y, row = blockIdx.x, tid = threadIdx.x;
  char* wr = reinterpret_cast<char*>(ws) + size_t(row) * bm_split_ws_per_row();
  int* count = reinterpret_cast<int*>(wr) + seg;
  uint32_t* wcode = reinterpret_cast<uint32_t*>(wr + 64) + size_t(seg) * kBmSegCap;
  int* widx = reinterpret_cast<int*>(wr + 64 + size_t(kBmSegs) * kBmSegCap * 4) +
              size_t(seg) * kBmSegCap;
  uint32_t* whist = reinterpret_cast<uint32_t*>(wr + 64 + size_t(kBmSegs) * kBmSegCap * 8) +
                    size_t(seg) * kBmSegBins;
  uint32_t* range = reinterpret_cast<uint32_t*>(wr) + kBmSegs;   // code(thr), row's largest
  if (tid < kBmSegBins) s_h[tid] = 0;                 // the barriers below order this
  const int lo = n_sink, hi = n - n_local, m = hi - lo;
  const int blo = lo / 64, nbc = m / 64;
  const int K = k < m ? k : m;
  const size_t base = size_t(row) * n;
  if (K == m || K == 0 || K > nbc) {                    // the final kernel takes the row path
    if (tid == 0) *count = -1;
    return;
  }
  const float* brow = bm + size_t(row) * nb + blo;
  float thr;
  uint32_t cmax;
  int nc = 0;
  if constexpr (GROUPS) {
    // groups wholly inside the competition blocks, and those meeting them
    const int gi0 = (blo + kBmGrp - 1) / kBmGrp, gi1 = (blo + nbc) / kBmGrp;
    const int gc0 = blo / kBmGrp, gc1 = (blo + nbc + kBmGrp - 1) / kBmGrp;
    // a contiguous eighth of the competition blocks; its maxima are loaded
    // with the group maxima (one round of loads)
    const int sb0 = int((long long)nbc * seg / kBmSegs), sb1 = int((long long)nbc * (seg + 1) / kBmSegs);
    float bv[kBmSegPer];
    load4_or_neg_inf(brow, sb0 + tid * kBmSegPer, sb1, bv);
    const int ngr = (nb + kBmGrp - 1) / kBmGrp;
    thr = bm_group_threshold(gm + size_t(row) * ngr, gi0, gi1, gc0, gc1, K, sbin, s_red, s_scan,
                             &s_thr, cmax);
    const int ncb = bm_list_blocks(bv, sb0, sb1, thr, cb, s_scan);
    if (ncb > 0)
      nc = bm_collect<4>(keys, base, blo, cb, ncb, thr, ckey, cidx, kBmSegCap, s_cnt, s_scan);
  } else {
    int ncb;
    if (!bm_candidate_blocks(brow, nbc, K, sbin, cb, s_red, s_scan, &s_thr, thr, ncb, cmax)) {
      if (tid == 0) *count = -1;
      return;
    }
    const int j0 = int((long long)ncb * seg / kBmSegs), j1 = int((long long)ncb * (seg + 1) / kBmSegs);
    if (j1 > j0)
      nc = bm_collect<4>(keys, base, blo, cb + j0, j1 - j0, thr, ckey, cidx, kBmSegCap, s_cnt, s_scan);
  }
  const uint32_t tc = s_thr;
  if (nc > kBmSegCap) {
    if (tid == 0) *count = -1;
    return;
  }
  for (int i = tid; i < nc; i += kTkThreads) {
    const uint32_t c = f32_order_key(ckey[i]);
    wcode[i] = c;
    widx[i] = cidx[i];
    atomicAdd(&s_h[bm_seg_bin(c - tc)], 1u);             // c >= tc: every candidate reaches thr
  }
  __syncthreads();
  if (tid < kBmSegBins) whist[tid] = s_h[tid];
  if (tid == 0) {
    *count = nc;
    if (seg == 0) {
      range[0] = tc;
      range[1] = cmax;
    }
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_bm_final_kernel(const float* __restrict__ keys,
                                                                   int n, int k, int n_sink,
                                                                   int n_local, const void* ws,
                                                                   int32_t* __restrict__ out,
                                                                   int stride) {
  __shared__ uint32_t ckey[kBmCap];
  __shared__ int cidx[kBmCap];
  __shared__ __align__(16) uint32_t hist[kKthHist];
  __shared__ uint32_t s_red[2 * kTkWaves];
  __shared__ int s_scan[4 * kTkWaves];
  __shared__ int s_bin, s_need;
  const int row = blockIdx.x, tid = threadIdx.x;
  int32_t* o = out + size_t(row) * stride;
  const char* wr = reinterpret_cast<const char*>(ws) + size_t(row) * bm_split_ws_per_row();
  const int* count = reinterpret_cast<const int*>(wr);
  const uint32_t* wcode = reinterpret_cast<const uint32_t*>(wr + 64);
  const int* widx = reinterpret_cast<const int*>(wr + 64 + size_t(kBmSegs) * kBmSegCap * 4);
  const uint32_t* whist = reinterpret_cast<const uint32_t*>(wr + 64 + size_t(kBmSegs) * kBmSegCap * 8);
  const uint32_t* range = reinterpret_cast<const uint32_t*>(wr) + kBmSegs;
  const int lo = n_sink, hi = n - n_local, m = hi - lo;
  const int K = k < m ? k : m;
  // one round of loads: every segment's count, and the first kFirst keys of
  // every segment (kTkThreads / kBmSegs threads a segment, two keys each);
  // the slots past a segment's count are read but not used
  constexpr int kTps = kTkThreads / kBmSegs;
  constexpr int kFirst = 2 * kTps;
  static_assert(kFirst <= kBmSegCap, "first round within a segment's slots");
  const int ms = tid / kTps, mj = 2 * (tid % kTps);
  const uint2 mc = *reinterpret_cast<const uint2*>(wcode + size_t(ms) * kBmSegCap + mj);
  const int2 mi = *reinterpret_cast<const int2*>(widx + size_t(ms) * kBmSegCap + mj);
  uint32_t hb = 0;                                    // bin tid summed over the segments
  if (tid < kBmSegBins) {
#pragma unroll
    for (int s = 0; s < kBmSegs; ++s) hb += whist[size_t(s) * kBmSegBins + tid];
  }
  const uint32_t tc = range[0], cmax = range[1];
  int cnt[kBmSegs], nc = 0;
  bool ok = true;
#pragma unroll
  for (int s = 0; s < kBmSegs; ++s) {
    cnt[s] = count[s];
    ok = ok && cnt[s] >= 0;
    nc += cnt[s] > 0 ? cnt[s] : 0;
  }
  if (!ok || nc > kBmCap || nc < K) {
    topk_row<SDQ_KEY_F32_MAX>(keys, size_t(row) * n, n, k, n_sink, n_local, o, stride);
    return;
  }
  // every segment's keys, segment after segment: index order again
  int moff = 0, mcnt = 0;
#pragma unroll
  for (int s = 0; s < kBmSegs; ++s) {
    moff += s < ms ? cnt[s] : 0;
    mcnt = s == ms ? cnt[s] : mcnt;
  }
  if (mj < mcnt) {
    ckey[moff + mj] = mc.x;
    cidx[moff + mj] = mi.x;
  }
  if (mj + 1 < mcnt) {
    ckey[moff + mj + 1] = mc.y;
    cidx[moff + mj + 1] = mi.y;
  }
  // the rest of segments longer than kFirst (rare)
  int off = 0;
#pragma unroll
  for (int s = 0; s < kBmSegs; ++s) {
    for (int i = kFirst + tid; i < cnt[s]; i += kTkThreads) {
      ckey[off + i] = wcode[size_t(s) * kBmSegCap + i];
      cidx[off + i] = widx[size_t(s) * kBmSegCap + i];
    }
    off += cnt[s];
  }
  // the bin holding the K-th largest candidate, from the summed histograms
  // (the exact search's first pass, already done by the segments)
  for (int i = tid; i < 2 * 256; i += kTkThreads) hist[i] = 0;
  {
    int tot;
    const int before = block_scan1<false>(int(hb), tot, s_scan);   // a barrier follows
    const int above = tot - before - int(hb);          // candidates in higher bins
    if (tid < kBmSegBins && above < K && above + int(hb) >= K) {
      s_bin = tid;
      s_need = K - above;
    }
  }
  __syncthreads();
  uint32_t boff, span;
  bm_seg_bin_range(uint32_t(s_bin), boff, span);
  const uint32_t blo = tc + boff;                       // <= cmax: the bin holds a candidate
  const uint32_t bhi = cmax - blo > span ? blo + span : cmax;
  const KthResult kr = select_kth_in(
      nc, s_need,
      [&](int i, uint32_t* u) {
        *u = ckey[i];
        return true;
      },
      hist, blo, bhi);
  bm_write_winners(ckey, cidx, nc, K, kr, n, n_sink, n_local, stride, o, s_scan);
}

}  // namespace sdq

using namespace sdq;

static bool use_fast(int n, int n_sink, int n_local, int k, int key_type) {
  const int m = n - n_sink - n_local;
  return key_type == SDQ_KEY_F32_MAX && m >= kFastMinComp && k < m && k <= kCandCap;
}

static bool use_block_max(int n, int n_sink, int n_local, int k, int key_type) {
  const int m = n - n_sink - n_local;
  return key_type == SDQ_KEY_F32_MAX && m >= kBmMinComp && n % 64 == 0 && n_sink % 64 == 0 &&
         n_local % 64 == 0 && n / 64 <= kBmMaxBlocks && k < m && k <= m / 64;
}

// uint8 rows long enough to split into segments (0 < k < competition length)
static bool use_u8_segments(int n, int n_sink, int n_local, int k) {
  const int m = n - n_sink - n_local;
  return m >= 2 * kU8Seg && k > 0 && k < m;
}

extern "C" size_t topk_select_workspace_bytes(int rows, int n, int k, int key_type) {
  if (rows < 1 || n < 1) return 0;
  (void)k;
  if (key_type == SDQ_KEY_U8_MIN && n >= 2 * kU8Seg)
    return size_t(rows) * cdiv(size_t(n), kU8Seg) * 256 * sizeof(uint32_t);
  if (key_type == SDQ_KEY_F32_MAX && n >= kFastMinComp) {
    const size_t hist = size_t(rows) * fast_ws_per_row();
    const size_t bm = size_t(rows) * size_t((n + 63) / 64) * sizeof(float);
    return hist > bm ? hist : bm;
  }
  return 256;
}

static int topk_validate(const char* nm, const void* keys, int key_type, int rows, int n, int k,
                         int n_sink, int n_local, const int32_t* idx_out, int* stride) {
  SDQ_REQUIRE(keys && idx_out, "%s: null pointer", nm);
  SDQ_REQUIRE(key_type == SDQ_KEY_F32_MAX || key_type == SDQ_KEY_U8_MIN,
              "%s: unknown key_type %d", nm, key_type);
  SDQ_REQUIRE(rows >= 1 && n >= 1, "%s: rows=%d, n=%d must be >= 1", nm, rows, n);
  SDQ_REQUIRE(k >= 0 && n_sink >= 0 && n_local >= 0, "%s: k, n_sink, n_local must be >= 0", nm);
  SDQ_REQUIRE(n_sink <= n - n_local, "%s: n_sink + n_local = %d exceeds n = %d", nm,
              n_sink + n_local, n);
  const long long stride_ll = (long long)k + n_sink + n_local;
  SDQ_REQUIRE(stride_ll <= 0x7FFFFFFF, "%s: output row too long", nm);
  *stride = int(stride_ll);
  return SDQ_OK;
}

static void launch_block_max_select(const float* fk, const float* bm, int rows, int n, int k,
                                    int n_sink, int n_local, int32_t* idx_out, int stride,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(topk_bm_kernel, dim3(rows), dim3(kTkThreads), 0, stream, fk, bm, n, n / 64, k,
                     n_sink, n_local, idx_out, stride);
}

// topk_select's launches over a given scratch buffer (the caller's workspace,
// or the library's static one for topk_select_noalloc).  Arguments are
// already validated; stride = k + n_sink + n_local > 0.
static int topk_select_launch(const char* nm, const void* keys, int key_type, int rows, int n, int k,
                              int n_sink, int n_local, int32_t* idx_out, int stride, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  const size_t need_ws = topk_select_workspace_bytes(rows, n, k, key_type);
  const float* fk = reinterpret_cast<const float*>(keys);
  if (use_block_max(n, n_sink, n_local, k, key_type) &&
      reinterpret_cast<uintptr_t>(keys) % 16 == 0) {
    SDQ_REQUIRE(ws && ws_bytes >= need_ws, "%s: workspace of %zu bytes needed, %zu given", nm,
                need_ws, ws_bytes);
    float* bm = reinterpret_cast<float*>(ws);
    const int nb = n / 64;
    hipLaunchKernelGGL(topk_block_max_kernel, dim3(cdiv(nb, 4), rows), dim3(256), 0, stream, fk, n,
                       nb, bm);
    launch_block_max_select(fk, bm, rows, n, k, n_sink, n_local, idx_out, stride, stream);
    return check_launch(nm);
  }
  if (use_fast(n, n_sink, n_local, k, key_type)) {
    SDQ_REQUIRE(ws && ws_bytes >= need_ws, "%s: workspace of %zu bytes needed, %zu given", nm,
                need_ws, ws_bytes);
    const int lo = n_sink, hi = n - n_local;
    dim3 g2(cdiv(hi - lo, kFastChunk), rows);
    hipLaunchKernelGGL(topk_clear_kernel, dim3(rows), dim3(256), 0, stream, ws);
    hipLaunchKernelGGL(topk_hist_kernel, g2, dim3(256), 0, stream, fk, n, lo, hi, ws);
    hipLaunchKernelGGL(topk_bin_kernel, dim3(rows), dim3(256), 0, stream, ws, k);
    hipLaunchKernelGGL(topk_collect_kernel, g2, dim3(256), 0, stream, fk, n, lo, hi, ws);
    hipLaunchKernelGGL(topk_final_kernel, dim3(rows), dim3(kTkThreads), 0, stream, fk, n, k, n_sink,
                       n_local, ws, idx_out, stride);
    return check_launch(nm);
  }
  if (key_type == SDQ_KEY_U8_MIN && use_u8_segments(n, n_sink, n_local, k)) {
    SDQ_REQUIRE(ws && ws_bytes >= need_ws, "%s: workspace of %zu bytes needed, %zu given", nm,
                need_ws, ws_bytes);
    const int lo = n_sink, hi = n - n_local;
    const int nseg = int(cdiv(size_t(hi - lo), kU8Seg));
    const uint8_t* u8 = reinterpret_cast<const uint8_t*>(keys);
    uint32_t* h = reinterpret_cast<uint32_t*>(ws);
    hipLaunchKernelGGL(topk_u8_hist_kernel, dim3(nseg, rows), dim3(kU8SegThreads), 0, stream, u8, n,
                       lo, hi, nseg, h);
    hipLaunchKernelGGL(topk_u8_select_kernel, dim3(nseg, rows), dim3(kU8SegThreads), 0, stream, u8,
                       n, k, n_sink, n_local, nseg, h, idx_out, stride);
    return check_launch(nm);
  }
  const int m_comp = n - n_sink - n_local;
  if (key_type == SDQ_KEY_F32_MAX && m_comp > kRowRegMin && m_comp <= kRowRegMax) {
    if (m_comp <= 2048)
      hipLaunchKernelGGL(topk_row_reg_kernel<2048>, dim3(rows), dim3(kTkThreads), 0, stream, fk, n,
                         k, n_sink, n_local, idx_out, stride);
    else if (m_comp <= 4096)
      hipLaunchKernelGGL(topk_row_reg_kernel<4096>, dim3(rows), dim3(kTkThreads), 0, stream, fk, n,
                         k, n_sink, n_local, idx_out, stride);
    else if (m_comp <= 8192)
      hipLaunchKernelGGL(topk_row_reg_kernel<8192>, dim3(rows), dim3(kTkThreads), 0, stream, fk, n,
                         k, n_sink, n_local, idx_out, stride);
    else if (m_comp <= 16384)
      hipLaunchKernelGGL(topk_row_reg_kernel<16384>, dim3(rows), dim3(kTkThreads), 0, stream, fk, n,
                         k, n_sink, n_local, idx_out, stride);
    else
      hipLaunchKernelGGL(topk_row_reg_kernel<kRowRegMax>, dim3(rows), dim3(kTkThreads), 0, stream,
                         fk, n, k, n_sink, n_local, idx_out, stride);
  } else if (key_type == SDQ_KEY_F32_MAX)
    hipLaunchKernelGGL(topk_row_kernel<SDQ_KEY_F32_MAX>, dim3(rows), dim3(kTkThreads), 0, stream,
                       keys, n, k, n_sink, n_local, idx_out, stride);
  else
    hipLaunchKernelGGL(topk_u8_kernel, dim3(rows), dim3(kTkThreads), 0, stream,
                       reinterpret_cast<const uint8_t*>(keys), n, k, n_sink, n_local, idx_out, stride);
  return check_launch(nm);
}


extern "C" int topk_select(const void* keys, int key_type, int rows, int n, int k, int n_sink,
                           int n_local, int32_t* idx_out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  int stride = 0;
  const int rc = topk_validate("topk_select", keys, key_type, rows, n, k, n_sink, n_local, idx_out,
                               &stride);
  if (rc != SDQ_OK) return rc;
  if (stride == 0) return SDQ_OK;
  return topk_select_launch("topk_select", keys, key_type, rows, n, k, n_sink, n_local, idx_out,
                            stride, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- no-allocation variant
// The scratch of topk_select_noalloc: one static array per GPU the library
// runs on, held until the process ends.  Host code never uses its name as an
// address (on the host it is only a stand-in for the symbol): the device
// address of each GPU's copy comes from hipGetSymbolAddress, once per device,
// and is what the kernels receive.
static __device__ __align__(256) uint8_t scratch[SDQ_TOPK_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of the current device's scratch, looked up on the first call
// on that device.  Returns SDQ_OK or SDQ_EHIP (message recorded).
static int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("topk_select_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    return SDQ_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("topk_select_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    return SDQ_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("topk_select_noalloc: hipGetSymbolAddress of the scratch failed on device %d: %s",
                dev, hipGetErrorString(e));
      return SDQ_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SDQ_OK;
}

extern "C" int topk_select_noalloc(const void* keys, int key_type, int rows, int n, int k,
                                   int n_sink, int n_local, int32_t* idx_out, hipStream_t stream) {
  int stride = 0;
  const int rc = topk_validate("topk_select_noalloc", keys, key_type, rows, n, k, n_sink, n_local,
                               idx_out, &stride);
  if (rc != SDQ_OK) return rc;
  const size_t need = topk_select_workspace_bytes(rows, n, k, key_type);
  SDQ_REQUIRE(need <= size_t(SDQ_TOPK_NOALLOC_SCRATCH_BYTES),
              "topk_select_noalloc: rows=%d x n=%d needs %zu bytes of scratch, the static scratch "
              "holds %zu (use topk_select with a workspace)",
              rows, n, need, size_t(SDQ_TOPK_NOALLOC_SCRATCH_BYTES));
  if (stride == 0) return SDQ_OK;
  void* ws = nullptr;
  const int rs = noalloc_scratch(&ws);
  if (rs != SDQ_OK) return rs;
  return topk_select_launch("topk_select_noalloc", keys, key_type, rows, n, k, n_sink, n_local,
                            idx_out, stride, ws, size_t(SDQ_TOPK_NOALLOC_SCRATCH_BYTES), stream);
}

extern "C" int hamming_scan(const uint32_t* sigs, const uint32_t* qsig, int H, int n, int n_cap,
                            uint8_t* dist, hipStream_t stream);

extern "C" int hamming_scan_topk(const uint32_t* sigs, const uint32_t* qsig, int H, int n, int n_cap,
                                 int k, int n_sink, int n_local, uint8_t* dist, int32_t* idx_out,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  SDQ_REQUIRE(sigs && qsig && dist, "hamming_scan_topk: null pointer");
  SDQ_REQUIRE(H >= 1 && n >= 1 && n <= n_cap, "hamming_scan_topk: H=%d, n=%d, n_cap=%d", H, n, n_cap);
  int stride = 0;
  const int rc = topk_validate("hamming_scan_topk", dist, SDQ_KEY_U8_MIN, H, n, k, n_sink, n_local,
                               idx_out, &stride);
  if (rc != SDQ_OK) return rc;
  if (!use_u8_segments(n, n_sink, n_local, k) || stride == 0) {
    const int r1 = hamming_scan(sigs, qsig, H, n, n_cap, dist, stream);
    if (r1 != SDQ_OK) return r1;
    return topk_select(dist, SDQ_KEY_U8_MIN, H, n, k, n_sink, n_local, idx_out, ws, ws_bytes, stream);
  }
  const size_t need_ws = topk_select_workspace_bytes(H, n, k, SDQ_KEY_U8_MIN);
  SDQ_REQUIRE(ws && ws_bytes >= need_ws,
              "hamming_scan_topk: workspace of %zu bytes needed, %zu given", need_ws, ws_bytes);
  const int lo = n_sink, hi = n - n_local;
  const int nseg = int(cdiv(size_t(hi - lo), kU8Seg));
  uint32_t* hst = reinterpret_cast<uint32_t*>(ws);
  hipLaunchKernelGGL(hamming_hist_kernel, dim3(nseg + 1, H), dim3(kHhThreads), 0, stream, sigs,
                     qsig, n, n_cap, lo, hi, nseg, dist, hst);
  hipLaunchKernelGGL(topk_u8_select_kernel, dim3(nseg, H), dim3(kU8SegThreads), 0, stream, dist, n,
                     k, n_sink, n_local, nseg, hst, idx_out, stride);
  return check_launch("hamming_scan_topk");
}

extern "C" int topk_select_block_max(const float* keys, const float* block_max, int rows, int n,
                                     int k, int n_sink, int n_local, int32_t* idx_out,
                                     hipStream_t stream) {
  int stride = 0;
  const int rc = topk_validate("topk_select_block_max", keys, SDQ_KEY_F32_MAX, rows, n, k, n_sink,
                               n_local, idx_out, &stride);
  if (rc != SDQ_OK) return rc;
  SDQ_REQUIRE(block_max, "topk_select_block_max: null block_max");
  SDQ_REQUIRE(n % 64 == 0 && n_sink % 64 == 0 && n_local % 64 == 0,
              "topk_select_block_max: n, n_sink and n_local must be multiples of 64");
  SDQ_REQUIRE(n / 64 <= kBmMaxBlocks, "topk_select_block_max: n=%d exceeds %d", n, kBmMaxBlocks * 64);
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(keys) % 16 == 0, "topk_select_block_max: keys must be 16-byte aligned");
  if (stride == 0) return SDQ_OK;
  launch_block_max_select(keys, block_max, rows, n, k, n_sink, n_local, idx_out, stride, stream);
  return check_launch("topk_select_block_max");
}

extern "C" size_t topk_select_block_max_split_workspace_bytes(int rows, int n) {
  if (rows < 1 || n < 1) return 0;
  return size_t(rows) * bm_split_ws_per_row();
}

extern "C" int topk_select_block_max_split(const float* keys, const float* block_max,
                                           const float* group_max, int rows, int n, int k,
                                           int n_sink, int n_local, int32_t* idx_out, void* ws,
                                           size_t ws_bytes, hipStream_t stream) {
  const char* nm = "topk_select_block_max_split";
  int stride = 0;
  const int rc = topk_validate(nm, keys, SDQ_KEY_F32_MAX, rows, n, k, n_sink, n_local, idx_out,
                               &stride);
  if (rc != SDQ_OK) return rc;
  SDQ_REQUIRE(block_max, "%s: null block_max", nm);
  SDQ_REQUIRE(n % 64 == 0 && n_sink % 64 == 0 && n_local % 64 == 0,
              "%s: n, n_sink and n_local must be multiples of 64", nm);
  SDQ_REQUIRE(n / 64 <= kBmMaxBlocks, "%s: n=%d exceeds %d", nm, n, kBmMaxBlocks * 64);
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(keys) % 16 == 0, "%s: keys must be 16-byte aligned", nm);
  SDQ_REQUIRE(rows <= 65535, "%s: rows=%d exceeds 65535", nm, rows);
  const size_t need = topk_select_block_max_split_workspace_bytes(rows, n);
  SDQ_REQUIRE(ws && ws_bytes >= need, "%s: workspace of %zu bytes needed, %zu given", nm, need,
              ws_bytes);
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(ws) % 16 == 0, "%s: ws must be 16-byte aligned", nm);
  if (stride == 0) return SDQ_OK;
  // the group maxima are used when at least K groups lie wholly inside the
  // competition blocks
  const int m = n - n_sink - n_local, K = k < m ? k : m;
  const int blo = n_sink / 64, bhi = (n - n_local) / 64;
  const bool groups = group_max && (bhi / kBmGrp) - (blo + kBmGrp - 1) / kBmGrp >= K;
  // grid (rows, segments): workgroups go round-robin over the XCDs by linear
  // id, so with rows a multiple of 8 the segments of row r share XCD r mod 8
  // with the final kernel's workgroup r, and the workspace they leave it
  // (and the row's maxima they all read) stays in that XCD's L2
  if (groups)
    hipLaunchKernelGGL(topk_bm_seg_kernel<true>, dim3(rows, kBmSegs), dim3(kTkThreads), 0, stream,
                       keys, block_max, group_max, n, n / 64, k, n_sink, n_local, ws);
  else
    hipLaunchKernelGGL(topk_bm_seg_kernel<false>, dim3(rows, kBmSegs), dim3(kTkThreads), 0, stream,
                       keys, block_max, nullptr, n, n / 64, k, n_sink, n_local, ws);
  hipLaunchKernelGGL(topk_bm_final_kernel, dim3(rows), dim3(kTkThreads), 0, stream, keys, n, k,
                     n_sink, n_local, ws, idx_out, stride);
  return check_launch(nm);
}
