// Shared device helpers and C-ABI error plumbing of libsdq (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/sdq.h"

namespace sdq {

constexpr int kWave = 64;
constexpr int kHeadDim = 128;

// ---------------------------------------------------------------- errors
void set_error(const char* fmt, ...);
void clear_error();

// Returns SDQ_EHIP (and records the message) if the last launch failed.
int check_launch(const char* what);

#define SDQ_REQUIRE(cond, ...)          \
  do {                                  \
    if (!(cond)) {                      \
      ::sdq::set_error(__VA_ARGS__);    \
      return SDQ_EINVAL;                \
    }                                   \
  } while (0)

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ float half_bits_to_f32(uint32_t h16) {
  return float(__builtin_bit_cast(_Float16, uint16_t(h16 & 0xFFFFu)));
}
__device__ __forceinline__ uint32_t f32_to_half_bits_rne(float x) {
  return uint32_t(__builtin_bit_cast(uint16_t, _Float16(x)));
}

__device__ __forceinline__ unsigned lane_id() { return __lane_id(); }

// Order-preserving map of a float32 to uint32 (larger float -> larger key).
// -0 is folded onto +0 first so that the two compare equal.
__device__ __forceinline__ uint32_t f32_order_key(float x) {
  uint32_t b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int m) {
  return __shfl_xor(v, m, kWave);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), in every lane of
// the row: quad swaps, then the half-row and row mirrors; no LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp_mov_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov_f32<0x141>(v);   // row_half_mirror: lane i <- lane 7-i of its half row
  v += dpp_mov_f32<0x140>(v);   // row_mirror: lane i <- lane 15-i of its row
  return v;
}

inline unsigned cdiv(size_t a, size_t b) { return unsigned((a + b - 1) / b); }

}  // namespace sdq
