// Offload mode of the plane index (Fathom summary, offload paragraph: the
// planes live in host memory, contiguous per channel, and before the scan one
// gather copies the active channels' plane prefixes into HBM at link rate).
//
// A zero-copy kernel reads the pinned, device-mapped host buffers over PCIe
// and writes the same offsets of an HBM staging copy.  The plan (depth) is
// read on the device, so the copy needs no host round trip and can run on a
// side stream ordered after the plan by an event.  Channel j of head g costs
// t_j*n/8 bytes of planes plus its n/64 metadata words; unread channels are
// not touched.
#include "common.hpp"

namespace sdq {

constexpr int kGaThreads = 256;
constexpr int kGaVecPerThread = 4;
constexpr int kGaChunkVec = kGaThreads * kGaVecPerThread;   // vectors per workgroup

template <typename V>
__global__ __launch_bounds__(kGaThreads) void fathom_gather_kernel(
    const V* __restrict__ planes_h, const uint32_t* __restrict__ meta_h,
    const uint8_t* __restrict__ depth, size_t plane_vecs, int nb64, int plane_chunks,
    V* __restrict__ planes_d, uint32_t* __restrict__ meta_d) {
  const int g = blockIdx.z, j = blockIdx.y;
  const int t = depth[size_t(g) * kHeadDim + j];
  if (t < 1 || t > 4) return;
  const size_t row = size_t(g) * kHeadDim + j;
  if (int(blockIdx.x) < plane_chunks) {
    const size_t len = size_t(t) * plane_vecs;               // prefix length in vectors
    const size_t base = row * 4 * plane_vecs;
    const size_t c0 = size_t(blockIdx.x) * kGaChunkVec;
    if (c0 >= len) return;
    V tmp[kGaVecPerThread];
#pragma unroll
    for (int e = 0; e < kGaVecPerThread; ++e) {
      const size_t i = c0 + size_t(e) * kGaThreads + threadIdx.x;
      if (i < len) tmp[e] = planes_h[base + i];
    }
#pragma unroll
    for (int e = 0; e < kGaVecPerThread; ++e) {
      const size_t i = c0 + size_t(e) * kGaThreads + threadIdx.x;
      if (i < len) planes_d[base + i] = tmp[e];
    }
  } else {
    const size_t c0 = size_t(int(blockIdx.x) - plane_chunks) * kGaChunkVec;
    for (int e = 0; e < kGaVecPerThread; ++e) {
      const size_t i = c0 + size_t(e) * kGaThreads + threadIdx.x;
      if (i < size_t(nb64)) meta_d[row * nb64 + i] = meta_h[row * nb64 + i];
    }
  }
}

}  // namespace sdq

using namespace sdq;

extern "C" int fathom_gather(const uint32_t* planes_host, const uint32_t* meta_host,
                             const uint8_t* depth, int G, int d, int n, uint32_t* planes_dev,
                             uint32_t* meta_dev, hipStream_t stream) {
  SDQ_REQUIRE(planes_host && meta_host && depth && planes_dev && meta_dev,
              "fathom_gather: null pointer");
  SDQ_REQUIRE(G >= 1, "fathom_gather: G=%d must be >= 1", G);
  SDQ_REQUIRE(n >= 64 && n % 64 == 0, "fathom_gather: n=%d must be a positive multiple of 64", n);
  SDQ_REQUIRE(d == kHeadDim, "fathom_gather: d=%d unsupported (only 128)", d);
  void* ph = nullptr;
  void* mh = nullptr;
  if (hipHostGetDevicePointer(&ph, const_cast<uint32_t*>(planes_host), 0) != hipSuccess || !ph ||
      hipHostGetDevicePointer(&mh, const_cast<uint32_t*>(meta_host), 0) != hipSuccess || !mh) {
    (void)hipGetLastError();
    sdq::set_error("fathom_gather: host buffers are not pinned device-mapped memory");
    return SDQ_EINVAL;
  }
  const int nb64 = n / 64;
  const size_t row_bytes = size_t(n) / 8;                    // one plane of one channel
  const int meta_chunks = cdiv(nb64, kGaChunkVec);
  const bool v16 = row_bytes % 16 == 0 && reinterpret_cast<uintptr_t>(ph) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(planes_dev) % 16 == 0;
  if (v16) {
    const size_t pv = row_bytes / 16;
    const int pc = cdiv(4 * pv, kGaChunkVec);
    dim3 grid(pc + meta_chunks, kHeadDim, G);
    hipLaunchKernelGGL(fathom_gather_kernel<uint4>, grid, dim3(kGaThreads), 0, stream,
                       reinterpret_cast<const uint4*>(ph), reinterpret_cast<const uint32_t*>(mh),
                       depth, pv, nb64, pc, reinterpret_cast<uint4*>(planes_dev), meta_dev);
  } else {
    const size_t pv = row_bytes / 8;
    const int pc = cdiv(4 * pv, kGaChunkVec);
    dim3 grid(pc + meta_chunks, kHeadDim, G);
    hipLaunchKernelGGL(fathom_gather_kernel<uint2>, grid, dim3(kGaThreads), 0, stream,
                       reinterpret_cast<const uint2*>(ph), reinterpret_cast<const uint32_t*>(mh),
                       depth, pv, nb64, pc, reinterpret_cast<uint2*>(planes_dev), meta_dev);
  }
  return check_launch("fathom_gather");
}
