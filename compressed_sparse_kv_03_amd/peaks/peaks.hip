// Measured ceilings: a streaming HBM read and independent MFMA chains (include/cskv_peaks.h).
#include <hip/hip_runtime.h>
#include <stdio.h>

#include "cskv.h"
#include "cskv_peaks.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadNT = 256;
constexpr int kMfmaNT = 256;
constexpr uint32_t kNever = 0x9E3779B9u;

thread_local char g_err[256];

int fail(int code, const char* msg) {
  snprintf(g_err, sizeof g_err, "%s", msg);
  return code;
}

// Grid-stride read: each thread requests eight 16-byte pieces (one stride apart, non-temporal)
// before using any.
constexpr int kReadU = 8;
__global__ __launch_bounds__(kReadNT) void peak_read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                            uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadNT;
  size_t i = (size_t)blockIdx.x * kReadNT + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadU - 1) * stride < n16; i += kReadU * stride) {
    u32x4 v[kReadU];
#pragma unroll
    for (int u = 0; u < kReadU; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == kNever) sink[blockIdx.x] = acc;
}

// Four independent accumulators per wave; operands fixed per lane (finite, small values).
template <int KIND>
__global__ __launch_bounds__(kMfmaNT) void peak_mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  if constexpr (KIND == 0) {
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
      b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
    }
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  } else {
    // KIND 1: e2m1 codes (cbsz = blgp = 4, the upper 4 dwords unused); KIND 2: e4m3 (0)
    constexpr int F = KIND == 1 ? 4 : 0;
    i32x8 a, b;
    for (int e = 0; e < 8; ++e) {
      const int v = KIND == 1 ? 0x12121212 : 0x30303030;  // small positive codes
      a[e] = (KIND == 1 && e >= 4) ? 0 : v + (lane & 1);
      b[e] = (KIND == 1 && e >= 4) ? 0 : v;
    }
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, F, F, 0, 127, 0, 127);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, F, F, 0, 127, 0, 127);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, F, F, 0, 127, 0, 127);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, F, F, 0, 127, 0, 127);
    }
  }
  float s = 0.f;
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == -1.f) sink[blockIdx.x] = s;  // the products are non-negative
}

}  // namespace

extern "C" CSKV_PEAKS_API const char* cskv_peaks_last_error(void) { return g_err; }

extern "C" CSKV_PEAKS_API int cskv_peak_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                                                 void* stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u) || bytes % 16 || bytes == 0)
    return fail(CSKV_EINVAL, "cskv_peak_hbm_read: null or misaligned buffer, or size not a positive multiple of 16");
  if (blocks < 1 || blocks > 65536) return fail(CSKV_EINVAL, "cskv_peak_hbm_read: blocks outside [1, 65536]");
  hipLaunchKernelGGL(peak_read_kernel, dim3(blocks), dim3(kReadNT), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4*>(buf), bytes / 16, sink);
  if (hipGetLastError() != hipSuccess) return fail(CSKV_EHIP, "cskv_peak_hbm_read: launch failed");
  return CSKV_OK;
}

extern "C" CSKV_PEAKS_API int cskv_peak_mfma(int kind, int iters, int blocks, float* sink, void* stream) {
  if (kind < 0 || kind > 2 || iters < 1 || blocks < 1 || blocks > 65536 || !sink)
    return fail(CSKV_EINVAL, "cskv_peak_mfma: kind outside [0, 2], iters < 1, blocks outside [1, 65536] or null sink");
  auto s = reinterpret_cast<hipStream_t>(stream);
  if (kind == 0) hipLaunchKernelGGL(peak_mfma_kernel<0>, dim3(blocks), dim3(kMfmaNT), 0, s, iters, sink);
  if (kind == 1) hipLaunchKernelGGL(peak_mfma_kernel<1>, dim3(blocks), dim3(kMfmaNT), 0, s, iters, sink);
  if (kind == 2) hipLaunchKernelGGL(peak_mfma_kernel<2>, dim3(blocks), dim3(kMfmaNT), 0, s, iters, sink);
  if (hipGetLastError() != hipSuccess) return fail(CSKV_EHIP, "cskv_peak_mfma: launch failed");
  return CSKV_OK;
}
