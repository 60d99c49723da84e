// Offload mode of the plane index (Fathom summary, offload paragraph: the
// planes live in host memory, contiguous per channel, and before the scan one
// gather copies the active channels' plane prefixes into HBM at link rate).
//
// A zero-copy kernel reads the pinned, device-mapped host buffers over PCIe
// and writes the same offsets of an HBM staging copy.  The plan (depth) is
// read on the device, so the copy needs no host round trip and can run on a
// side stream ordered after the plan by an event.  Channel j of head g costs
// t_j*n/8 bytes of planes plus its n/64 metadata words (n rounded up to 64);
// unread channels are not touched.
#include "common.hpp"

namespace sdq {

constexpr int kGaThreads = 256;
constexpr int kGaVecPerThread = 4;
constexpr int kGaChunkVec = kGaThreads * kGaVecPerThread;   // vectors per workgroup

// Grid: x = 4 planes x `cpp` chunks of one plane's prefix, then the metadata
// chunks; y = channel; z = KV head.  Plane rows are `row_vecs` vectors apart
// (the row capacity) and `len_vecs` of each are copied (the tokens scored,
// rounded up to 64); metadata rows are nb_cap words apart, nb of them copied.
template <typename V>
__global__ __launch_bounds__(kGaThreads) void fathom_gather_kernel(
    const V* __restrict__ planes_h, const uint32_t* __restrict__ meta_h,
    const uint8_t* __restrict__ depth, size_t row_vecs, size_t len_vecs, int cpp, int nb,
    int nb_cap, V* __restrict__ planes_d, uint32_t* __restrict__ meta_d) {
  const int g = blockIdx.z, j = blockIdx.y;
  const int t = depth[size_t(g) * kHeadDim + j];
  if (t < 1 || t > 4) return;
  const size_t row = size_t(g) * kHeadDim + j;
  if (int(blockIdx.x) < 4 * cpp) {
    const int p = int(blockIdx.x) / cpp;                      // plane of this chunk
    if (p >= t) return;
    const size_t base = (row * 4 + p) * row_vecs;
    const size_t c0 = size_t(int(blockIdx.x) - p * cpp) * kGaChunkVec;
    V tmp[kGaVecPerThread];
#pragma unroll
    for (int e = 0; e < kGaVecPerThread; ++e) {
      const size_t i = c0 + size_t(e) * kGaThreads + threadIdx.x;
      if (i < len_vecs) tmp[e] = planes_h[base + i];
    }
#pragma unroll
    for (int e = 0; e < kGaVecPerThread; ++e) {
      const size_t i = c0 + size_t(e) * kGaThreads + threadIdx.x;
      if (i < len_vecs) planes_d[base + i] = tmp[e];
    }
  } else {
    const size_t c0 = size_t(int(blockIdx.x) - 4 * cpp) * kGaChunkVec;
    for (int e = 0; e < kGaVecPerThread; ++e) {
      const size_t i = c0 + size_t(e) * kGaThreads + threadIdx.x;
      if (i < size_t(nb)) meta_d[row * nb_cap + i] = meta_h[row * nb_cap + i];
    }
  }
}

}  // namespace sdq

using namespace sdq;

extern "C" int fathom_gather(const uint32_t* planes_host, const uint32_t* meta_host,
                             const uint8_t* depth, int G, int d, int n, int n_cap,
                             uint32_t* planes_dev, uint32_t* meta_dev, hipStream_t stream) {
  SDQ_REQUIRE(planes_host && meta_host && depth && planes_dev && meta_dev,
              "fathom_gather: null pointer");
  SDQ_REQUIRE(G >= 1, "fathom_gather: G=%d must be >= 1", G);
  SDQ_REQUIRE(n_cap >= 64 && n_cap % 64 == 0 && n_cap < (1 << 25),
              "fathom_gather: n_cap=%d must be a positive multiple of 64 below 2^25", n_cap);
  SDQ_REQUIRE(n >= 1 && n <= n_cap, "fathom_gather: n=%d must be in [1, n_cap=%d]", n, n_cap);
  SDQ_REQUIRE(d == kHeadDim, "fathom_gather: d=%d unsupported (only 128)", d);
  void* ph = nullptr;
  void* mh = nullptr;
  if (hipHostGetDevicePointer(&ph, const_cast<uint32_t*>(planes_host), 0) != hipSuccess || !ph ||
      hipHostGetDevicePointer(&mh, const_cast<uint32_t*>(meta_host), 0) != hipSuccess || !mh) {
    (void)hipGetLastError();
    sdq::set_error("fathom_gather: host buffers are not pinned device-mapped memory");
    return SDQ_EINVAL;
  }
  const int nb = (n + 63) / 64;                              // blocks scored
  const size_t row_bytes = size_t(n_cap) / 8;                // one plane row of one channel
  const size_t len_bytes = size_t(nb) * 8;                   // its scored prefix
  const int meta_chunks = cdiv(nb, kGaChunkVec);
  const bool v16 = row_bytes % 16 == 0 && len_bytes % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(ph) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(planes_dev) % 16 == 0;
  if (v16) {
    const int cpp = cdiv(len_bytes / 16, kGaChunkVec);
    dim3 grid(4 * cpp + meta_chunks, kHeadDim, G);
    hipLaunchKernelGGL(fathom_gather_kernel<uint4>, grid, dim3(kGaThreads), 0, stream,
                       reinterpret_cast<const uint4*>(ph), reinterpret_cast<const uint32_t*>(mh),
                       depth, row_bytes / 16, len_bytes / 16, cpp, nb, n_cap / 64,
                       reinterpret_cast<uint4*>(planes_dev), meta_dev);
  } else {
    const int cpp = cdiv(len_bytes / 8, kGaChunkVec);
    dim3 grid(4 * cpp + meta_chunks, kHeadDim, G);
    hipLaunchKernelGGL(fathom_gather_kernel<uint2>, grid, dim3(kGaThreads), 0, stream,
                       reinterpret_cast<const uint2*>(ph), reinterpret_cast<const uint32_t*>(mh),
                       depth, row_bytes / 8, len_bytes / 8, cpp, nb, n_cap / 64,
                       reinterpret_cast<uint2*>(planes_dev), meta_dev);
  }
  return check_launch("fathom_gather");
}
