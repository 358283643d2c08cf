// Device helpers shared by the gfx950 kernels: storage conversions, wave-level
// reductions, RoPE angles. Wavefront size is 64 on CDNA4.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cskv {

constexpr int kWave = 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: data read once).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// 8 bf16 in a uint4 -> 8 floats
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

// ---------------------------------------------------------------- fp8 e4m3fn (OCP)
// gfx950's v_cvt_*fp8* instructions use the OCP e4m3fn encoding.
__device__ __forceinline__ float fp8_to_f32(uint32_t word, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(word, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(word, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(word, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(word, 3);
  }
}
// four fp32 -> four e4m3fn codes (RNE), packed little-endian
__device__ __forceinline__ uint32_t f32x4_to_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------- wave reductions
// Reductions over the 16 lanes of each DPP row (lanes 16r..16r+15); every lane gets the
// result. quad_perm [1,0,3,2] and [2,3,0,1] combine within quads, row_ror 4 and 8 across them.
__device__ __forceinline__ int dpp_i(int x, int ctrl) {
  switch (ctrl) {
    case 0: return __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);
    case 1: return __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false);
    default: return __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false);
  }
}
__device__ __forceinline__ float dpp_f(float v, int ctrl) {
  return __builtin_bit_cast(float, dpp_i(__builtin_bit_cast(int, v), ctrl));
}
__device__ __forceinline__ double dpp_d(double v, int ctrl) {
  const uint64_t x = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)dpp_i((int)(uint32_t)x, ctrl), hi = (uint32_t)dpp_i((int)(uint32_t)(x >> 32), ctrl);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f(v, 0));
  v = fmaxf(v, dpp_f(v, 1));
  v = fmaxf(v, dpp_f(v, 2));
  return fmaxf(v, dpp_f(v, 3));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f(v, 0);
  v += dpp_f(v, 1);
  v += dpp_f(v, 2);
  return v + dpp_f(v, 3);
}
// Whole-wave reductions: the four row results read with readlane (every lane gets the result;
// no LDS round trip as for shuffles).
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ double lane_d(double v, int l) {
  const uint64_t x = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v = fmax(v, dpp_d(v, c));
  return fmax(fmax(lane_d(v, 0), lane_d(v, 16)), fmax(lane_d(v, 32), lane_d(v, 48)));
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v += dpp_d(v, c);
  return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}

// ---------------------------------------------------------------- RoPE
// Angle p * base^(-2i/d_rope), formed in fp64 and reduced to [-pi, pi] before
// the fp32 rotation (positions reach 2^20, where an fp32 angle would be off by
// up to ~0.06 rad).
__device__ __forceinline__ double rope_inv_freq(float base, int pair, int d_rope) {
  return pow((double)base, -2.0 * (double)pair / (double)d_rope);
}

}  // namespace cskv
