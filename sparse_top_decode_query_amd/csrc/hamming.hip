// Hamming distances of packed 32-bit signatures (HashAttention study notes,
// sec. 2.2: score = -popcount(h_i XOR h_q)).  HBM-bound streaming kernel:
// 4 bytes read and 1 byte written per token-head; each lane handles 16
// consecutive signatures (one 64-byte read, one 16-byte write).  Signature
// rows hold n_cap tokens (a growing cache's capacity), the first n scored.
#include "common.hpp"

namespace sdq {

__global__ __launch_bounds__(256) void hamming_scan_vec_kernel(const uint4* __restrict__ sigs,
                                                               const uint32_t* __restrict__ qsig,
                                                               int n16, int cap16,
                                                               uint4* __restrict__ dist) {
  const int h = blockIdx.y;
  const uint32_t qs = qsig[h];
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n16) return;
  const uint4* src = sigs + (size_t(h) * cap16 + i) * 4;
  uint32_t outw[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint4 s = src[v];
    outw[v] = uint32_t(__popc(s.x ^ qs)) | (uint32_t(__popc(s.y ^ qs)) << 8) |
              (uint32_t(__popc(s.z ^ qs)) << 16) | (uint32_t(__popc(s.w ^ qs)) << 24);
  }
  dist[size_t(h) * n16 + i] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
}

__global__ __launch_bounds__(256) void hamming_scan_kernel(const uint32_t* __restrict__ sigs,
                                                           const uint32_t* __restrict__ qsig, int n,
                                                           int n_cap, uint8_t* __restrict__ dist) {
  const int h = blockIdx.y;
  const uint32_t qs = qsig[h];
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    dist[size_t(h) * n + i] = uint8_t(__popc(sigs[size_t(h) * n_cap + i] ^ qs));
}

}  // namespace sdq

using namespace sdq;

extern "C" int hamming_scan(const uint32_t* sigs, const uint32_t* qsig, int H, int n, int n_cap,
                            uint8_t* dist, hipStream_t stream) {
  SDQ_REQUIRE(sigs && qsig && dist, "hamming_scan: null pointer");
  SDQ_REQUIRE(H >= 1 && n >= 1, "hamming_scan: H=%d, n=%d must be >= 1", H, n);
  SDQ_REQUIRE(n <= n_cap, "hamming_scan: n=%d exceeds n_cap=%d", n, n_cap);
  const bool aligned = (reinterpret_cast<uintptr_t>(sigs) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(dist) % 16 == 0);
  if (n % 16 == 0 && n_cap % 16 == 0 && aligned) {
    const int n16 = n / 16;
    dim3 grid(cdiv(n16, 256), H);
    hipLaunchKernelGGL(hamming_scan_vec_kernel, grid, dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(sigs), qsig, n16, n_cap / 16,
                       reinterpret_cast<uint4*>(dist));
  } else {
    const unsigned bx = cdiv(n, 256) < 1024u ? cdiv(n, 256) : 1024u;
    dim3 grid(bx, H);
    hipLaunchKernelGGL(hamming_scan_kernel, grid, dim3(256), 0, stream, sigs, qsig, n, n_cap, dist);
  }
  return check_launch("hamming_scan");
}
