// KV selection against a GPU-resident block pool, and the planned block fetch
// (OasisKV review: core method and method-steps sections).
//
// Each (request, KV head) row keeps S slots of resident blocks.  A step's
// predicted block set P (the top-K under the draft query) is intersected with
// the pool: hits stay and are stamped with the step; predicted blocks that are
// not resident (misses, best score first, equal scores to the lower block id)
// are paired with eviction targets (empty slots first, then occupied slots
// whose block is not in P by last-selected step ascending, equal stamps to the
// lower slot), at most `cap` pairs per row.  The pairs are the step's transfer
// plan; oasis_fetch then copies each planned block from pinned host memory
// into its slot over the host link (zero-copy reads, as fathom_gather).
//
// One workgroup per row.  P and the resident blocks become two bitmaps over
// the row's nb blocks in LDS, so membership is one LDS read; misses and
// targets are compacted into LDS and each one's rank is counted against all
// the others (at most 1024 of each, so at most 4 passes of 256 threads over
// 1024 candidates).
#include "common.hpp"

namespace sdq {

constexpr int kOsThreads = 256;
constexpr int kOsMaxK = 1024;            // predicted blocks per row
constexpr int kOsMaxS = 1024;            // slots per row
constexpr int kOsMaxBlocks = 1 << 16;    // blocks per row (two 8 KB bitmaps)

__device__ __forceinline__ bool bit_of(const uint32_t* bm, int b) {
  return (bm[b >> 5] >> (b & 31)) & 1u;
}

__global__ __launch_bounds__(kOsThreads) void oasis_select_kernel(
    const int32_t* __restrict__ pred, int K, const float* __restrict__ scores, int nb,
    int32_t* __restrict__ resident, int32_t* __restrict__ last_sel, int S, int step, int cap,
    int32_t* __restrict__ plan_slot, int32_t* __restrict__ plan_block,
    int32_t* __restrict__ n_fetch, int32_t* __restrict__ slots_out) {
  __shared__ uint32_t s_pred[kOsMaxBlocks / 32];
  __shared__ uint32_t s_held[kOsMaxBlocks / 32];
  __shared__ int s_miss[kOsMaxK];        // compacted misses: block id
  __shared__ float s_msc[kOsMaxK];       //   and its score
  __shared__ int s_targ[kOsMaxS];        // compacted targets: slot
  __shared__ int s_tkey[kOsMaxS];        //   occupied ? stamp : (empty)
  __shared__ int s_tocc[kOsMaxS];
  __shared__ int s_mb[kOsMaxK];          // miss of rank r
  __shared__ int s_ts[kOsMaxS];          // target of rank r
  __shared__ int s_occ[kOsMaxS];         // slot holds a block after the step
  __shared__ int s_nmiss, s_ntarg;
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int nwords = (nb + 31) >> 5;
  const int32_t* prow = pred + size_t(r) * K;
  int32_t* res = resident + size_t(r) * S;
  int32_t* ls = last_sel + size_t(r) * S;
  const float* sc = scores + size_t(r) * nb;

  for (int w = t; w < nwords; w += kOsThreads) {
    s_pred[w] = 0u;
    s_held[w] = 0u;
  }
  for (int i = t; i < kOsMaxK; i += kOsThreads) s_mb[i] = -1;   // ranks left unfilled read as
  for (int i = t; i < kOsMaxS; i += kOsThreads) s_ts[i] = -1;   // "no pair" (NaN scores only)
  if (t == 0) {
    s_nmiss = 0;
    s_ntarg = 0;
  }
  __syncthreads();
  for (int k = t; k < K; k += kOsThreads) {
    const int b = prow[k];
    if (b >= 0 && b < nb) atomicOr(&s_pred[b >> 5], 1u << (b & 31));
  }
  for (int s = t; s < S; s += kOsThreads) {
    const int b = res[s];
    if (b >= 0 && b < nb) atomicOr(&s_held[b >> 5], 1u << (b & 31));
  }
  __syncthreads();
  // hits are stamped; every other slot is an eviction target
  for (int s = t; s < S; s += kOsThreads) {
    const int b = res[s];
    s_occ[s] = b >= 0;
    if (b >= 0 && b < nb && bit_of(s_pred, b)) {
      ls[s] = step;
    } else {
      const int pos = atomicAdd(&s_ntarg, 1);
      s_targ[pos] = s;
      s_tocc[pos] = b >= 0;
      s_tkey[pos] = b >= 0 ? ls[s] : 0;
    }
  }
  // a miss is claimed by setting its bit in the resident bitmap, so a block
  // listed twice in P is listed once here
  for (int k = t; k < K; k += kOsThreads) {
    const int b = prow[k];
    if (b >= 0 && b < nb && !(atomicOr(&s_held[b >> 5], 1u << (b & 31)) & (1u << (b & 31)))) {
      const int pos = atomicAdd(&s_nmiss, 1);
      s_miss[pos] = b;
      s_msc[pos] = sc[b];
    }
  }
  __syncthreads();
  const int M = s_nmiss, T = s_ntarg;
  // rank = number of candidates that come first (the orders are total)
  for (int i = t; i < M; i += kOsThreads) {
    const int b = s_miss[i];
    const float v = s_msc[i];
    int rank = 0;
    for (int j = 0; j < M; ++j) {
      const float u = s_msc[j];
      rank += (u > v) || (u == v && s_miss[j] < b);
    }
    s_mb[rank] = b;
  }
  for (int i = t; i < T; i += kOsThreads) {
    const int s = s_targ[i], o = s_tocc[i], key = s_tkey[i];
    int rank = 0;
    for (int j = 0; j < T; ++j) {
      const int oj = s_tocc[j], kj = s_tkey[j];
      rank += (oj < o) || (oj == o && (kj < key || (kj == key && s_targ[j] < s)));
    }
    s_ts[rank] = s;
  }
  __syncthreads();
  const int m = min(cap, min(M, T));
  for (int i = t; i < cap; i += kOsThreads) {
    int s = -1, b = -1;
    if (i < m && s_ts[i] >= 0 && s_mb[i] >= 0) {
      s = s_ts[i];
      b = s_mb[i];
      res[s] = b;
      ls[s] = step;
      s_occ[s] = 1;
    }
    plan_slot[size_t(r) * cap + i] = s;
    plan_block[size_t(r) * cap + i] = b;
  }
  if (t == 0) n_fetch[r] = m;
  if (slots_out) {
    __syncthreads();
    for (int s = t; s < S; s += kOsThreads) slots_out[size_t(r) * S + s] = s_occ[s] ? s : -1;
  }
}

// One workgroup per planned pair: block b of the row's host cache (rows of
// `bt` tokens x 256 bytes, K and V) goes to slot s of the row's pool.
__global__ __launch_bounds__(kOsThreads) void oasis_fetch_kernel(
    const uint4* __restrict__ K_src, const uint4* __restrict__ V_src,
    const int32_t* __restrict__ plan_slot, const int32_t* __restrict__ plan_block, int cap, int nb,
    int bt, int S, uint4* __restrict__ K_pool, uint4* __restrict__ V_pool) {
  const int i = blockIdx.x, r = blockIdx.y;
  const int s = plan_slot[size_t(r) * cap + i];
  const int b = plan_block[size_t(r) * cap + i];
  if (s < 0 || s >= S || b < 0 || b >= nb) return;
  const int nv = bt * (kHeadDim / 8);                        // 16-byte vectors per block
  const size_t src = (size_t(r) * nb + b) * nv;
  const size_t dst = (size_t(r) * S + s) * nv;
  for (int v = threadIdx.x; v < nv; v += kOsThreads) {
    const uint4 kv = K_src[src + v];
    const uint4 vv = V_src[src + v];
    K_pool[dst + v] = kv;
    V_pool[dst + v] = vv;
  }
}

}  // namespace sdq

using namespace sdq;

extern "C" int oasis_select(const int32_t* pred, int K, const float* block_scores, int nb, int rows,
                            int32_t* resident, int32_t* last_sel, int S, int step, int cap,
                            int32_t* plan_slot, int32_t* plan_block, int32_t* n_fetch,
                            int32_t* slots_out, hipStream_t stream) {
  SDQ_REQUIRE(resident && last_sel && n_fetch, "oasis_select: null pointer");
  SDQ_REQUIRE(K == 0 || (pred && block_scores), "oasis_select: null pointer");
  SDQ_REQUIRE(cap == 0 || (plan_slot && plan_block), "oasis_select: null pointer");
  SDQ_REQUIRE(rows >= 1, "oasis_select: rows=%d must be >= 1", rows);
  SDQ_REQUIRE(K >= 0 && K <= kOsMaxK, "oasis_select: K=%d outside [0, %d]", K, kOsMaxK);
  SDQ_REQUIRE(S >= 1 && S <= kOsMaxS, "oasis_select: S=%d outside [1, %d]", S, kOsMaxS);
  SDQ_REQUIRE(nb >= 1 && nb <= kOsMaxBlocks, "oasis_select: nb=%d outside [1, %d]", nb, kOsMaxBlocks);
  SDQ_REQUIRE(cap >= 0 && cap <= kOsMaxS, "oasis_select: cap=%d outside [0, %d]", cap, kOsMaxS);
  hipLaunchKernelGGL(oasis_select_kernel, dim3(rows), dim3(kOsThreads), 0, stream, pred, K,
                     block_scores, nb, resident, last_sel, S, step, cap, plan_slot, plan_block,
                     n_fetch, slots_out);
  return check_launch("oasis_select");
}

extern "C" int oasis_fetch(const uint16_t* K_host, const uint16_t* V_host, const int32_t* plan_slot,
                           const int32_t* plan_block, int rows, int cap, int nb, int block_tokens,
                           int d, uint16_t* K_pool, uint16_t* V_pool, int S, hipStream_t stream) {
  SDQ_REQUIRE(K_host && V_host && K_pool && V_pool, "oasis_fetch: null pointer");
  SDQ_REQUIRE(cap == 0 || (plan_slot && plan_block), "oasis_fetch: null pointer");
  SDQ_REQUIRE(rows >= 1 && nb >= 1 && S >= 1 && block_tokens >= 1 && cap >= 0,
              "oasis_fetch: rows, nb, S, block_tokens must be >= 1 and cap >= 0");
  SDQ_REQUIRE(d == kHeadDim, "oasis_fetch: d=%d unsupported (only 128)", d);
  SDQ_REQUIRE((long long)nb * block_tokens <= (1LL << 24) && (long long)S * block_tokens <= (1LL << 24),
              "oasis_fetch: more than 2^24 tokens per row");
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(K_pool) % 16 == 0 && reinterpret_cast<uintptr_t>(V_pool) % 16 == 0,
              "oasis_fetch: pools must be 16-byte aligned");
  if (cap == 0) return SDQ_OK;
  void* kd = nullptr;
  void* vd = nullptr;
  if (hipHostGetDevicePointer(&kd, const_cast<uint16_t*>(K_host), 0) != hipSuccess || !kd ||
      hipHostGetDevicePointer(&vd, const_cast<uint16_t*>(V_host), 0) != hipSuccess || !vd) {
    (void)hipGetLastError();
    set_error("oasis_fetch: K_host and V_host must be pinned, device-mapped host memory");
    return SDQ_EINVAL;
  }
  SDQ_REQUIRE(reinterpret_cast<uintptr_t>(kd) % 16 == 0 && reinterpret_cast<uintptr_t>(vd) % 16 == 0,
              "oasis_fetch: host caches must be 16-byte aligned");
  hipLaunchKernelGGL(oasis_fetch_kernel, dim3(cap, rows), dim3(kOsThreads), 0, stream,
                     static_cast<const uint4*>(kd), static_cast<const uint4*>(vd), plan_slot,
                     plan_block, cap, nb, block_tokens, S, reinterpret_cast<uint4*>(K_pool),
                     reinterpret_cast<uint4*>(V_pool));
  return check_launch("oasis_fetch");
}
