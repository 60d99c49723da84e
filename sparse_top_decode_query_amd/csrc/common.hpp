// Shared device helpers and C-ABI error plumbing of libsdq (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/sdq.h"

namespace sdq {

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

__device__ __forceinline__ float half_bits_to_f32(uint32_t h16) {
  return float(__builtin_bit_cast(_Float16, uint16_t(h16 & 0xFFFFu)));
}
__device__ __forceinline__ uint32_t f32_to_half_bits_rne(float x) {
  return uint32_t(__builtin_bit_cast(uint16_t, _Float16(x)));
}

// Order-preserving map of a float32 to uint32 (larger float -> larger key).
// -0 is folded onto +0 first so that the two compare equal.
__device__ __forceinline__ uint32_t f32_order_key(float x) {
  uint32_t b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
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

// DPP scans and reductions (no LDS traffic).  A DPP lane whose source lane
// does not exist, or whose row is masked off, receives 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
// Inclusive prefix sum within each 16-lane row.
__device__ __forceinline__ int row16_incl_scan(int x) {
  x += dpp_i32<0x111>(x);         // row_shr:1
  x += dpp_i32<0x112>(x);         // row_shr:2
  x += dpp_i32<0x114>(x);         // row_shr:4
  x += dpp_i32<0x118>(x);         // row_shr:8
  return x;
}
// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x = row16_incl_scan(x);
  x += dpp_i32<0x142, 0xA>(x);    // row_bcast:15 into rows 1 and 3
  x += dpp_i32<0x143, 0xC>(x);    // row_bcast:31 into rows 2 and 3
  return x;
}
// Value of lane 63, as a wave-uniform scalar.
__device__ __forceinline__ int wave_last(int x) { return __builtin_amdgcn_readlane(x, 63); }
// Sum over the wave, wave-uniform.
__device__ __forceinline__ int wave_sum_dpp(int x) { return wave_last(wave_incl_scan(x)); }
// Min / max over the wave of unsigned values, wave-uniform: within rows by
// DPP, then the four row results by lane reads.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
  auto f = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = f(v, uint32_t(dpp_i32<0xB1>(int(v))));     // quad_perm [1,0,3,2]
  v = f(v, uint32_t(dpp_i32<0x4E>(int(v))));     // quad_perm [2,3,0,1]
  v = f(v, uint32_t(dpp_i32<0x141>(int(v))));    // row_half_mirror
  v = f(v, uint32_t(dpp_i32<0x140>(int(v))));    // row_mirror
  const uint32_t r0 = uint32_t(__builtin_amdgcn_readlane(int(v), 0));
  const uint32_t r1 = uint32_t(__builtin_amdgcn_readlane(int(v), 16));
  const uint32_t r2 = uint32_t(__builtin_amdgcn_readlane(int(v), 32));
  const uint32_t r3 = uint32_t(__builtin_amdgcn_readlane(int(v), 48));
  return f(f(r0, r1), f(r2, r3));
}

inline unsigned cdiv(size_t a, size_t b) { return unsigned((a + b - 1) / b); }

}  // namespace sdq
