// KV compression (softmax pooling of m-token blocks + partial RoPE + storage
// rounding) and the decode-time ring append.
//
// Method: page "DeepSeek-V4가 이차적 어텐션 비용 없이 백만 토큰 컨텍스트를 달성하는
// 방법", section "두 가지 압축 전략: CSA 및 HCA" (4 tokens per CSA entry, 128 per
// HCA entry, softmax-weighted pooling, partial RoPE); page "딥시크 V4 분석:
// CSA·HCA 어텐션으로 100만 토큰 컨텍스트를 저비용에 구현한 방법", section "쉽게
// 이해하기" (per-token learned contribution; 128-token window).
//
// Design (HBM-bound stream): one wavefront per output entry. Lane l owns the
// 16-byte chunks l and l+64 of the D-dim row, so each token row is read by one
// coalesced 1 KiB wave load (+ a short tail when D > 512). The arithmetic is
// fp64 from the bf16 inputs to the storage rounding (pooling weights, pooled
// sums, RMSNorm, the RoPE angle and its sine and cosine, the fp8 scale), and
// the stored value is rounded once, from fp64, to its format: the stored entry
// is then the correct rounding of the exact entry except where the exact value
// lies within a few fp64 ulps of a rounding midpoint. fp64 runs at half the
// fp32 vector rate on this GPU, far above what a stream of bf16 tokens needs.
// The m pooling weights are computed once per token into the wave's LDS slot
// and read back as wave-uniform values; the fp8 scale needs the entry's
// max |e|, a wave reduction with no LDS and no barrier.
#include "common.cuh"
#include "host_util.h"

namespace cskv {

constexpr int kCompressWaves = 4;  // waves per workgroup
constexpr int kUnroll = 8;
constexpr int kRopeTab = 64;       // RoPE pairs whose frequency comes from the host table
constexpr int kMaxBlock = 1024;    // largest m

// base^(-2i/d_rope) for the first kRopeTab pairs, formed on the host in fp64 (a device fp64
// pow per pair and lane was most of the kernel's time at decode sizes).
struct RopeTable {
  double inv_freq[kRopeTab];
};

// floor(log2 |v|) of a finite nonzero double (exact: from the binary exponent).
__device__ __forceinline__ int floor_log2_d(double v) {
  int ex;
  (void)frexp(v, &ex);  // |v| = f * 2^ex with f in [0.5, 1)
  return ex - 1;
}

// fp64 -> bf16 bits, round to nearest even (finite values in the bf16 range; +-0 -> 0).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
  if (v == 0.0) return 0u;
  const int e = max(floor_log2_d(v), -126);
  const double r = ldexp(rint(ldexp(v, 7 - e)), e - 7);  // 8 significant bits; scalings exact
  return __float_as_uint((float)r) >> 16;              // exact: r has 8 significant bits
}

// fp64 -> OCP e4m3fn code: round to nearest even on 4 significant bits (quantum 2^-9 below
// 2^-6), saturating at 448; a strictly negative value keeps the sign bit when it rounds to 0.
__device__ __forceinline__ uint32_t f64_to_e4m3(double v) {
  const double a = fabs(v);
  int code = 0;
  if (a > 0.0) {
    const int e = max(floor_log2_d(a), -6);
    const int r = (int)rint(ldexp(a, 3 - e));  // in [0, 16]; 16 carries into the next binade
    code = min((e + 7) * 8 + r - 8, 0x7E);      // e = -6 gives code = r (subnormals, 2^-6)
  }
  return (uint32_t)code | (v < 0.0 ? 0x80u : 0u);
}

// Nearest e2m1 code of v in units of the block scale (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
// ties to the even code, saturating at 6), sign in bit 3 for a strictly negative value.
__device__ __forceinline__ uint32_t e2m1_code_d(double v) {
  const double mag = fabs(v);
  const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  int c = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) c += mag > mids[i];
  bool tie = false;
#pragma unroll
  for (int i = 0; i < 7; ++i) tie = tie || (c == i && mag == mids[i]);
  if (tie && (c & 1)) ++c;  // a midpoint goes to the even code
  return (uint32_t)c | (v < 0.0 ? 8u : 0u);
}

// MXFP4 block exponent of a block whose largest magnitude is amax: floor(log2 amax) - 2 (the
// largest e2m1 exponent) limited to [e_min, e_max]; an all-zero block takes e_min.
__device__ __forceinline__ int mx_block_exp(double amax, int e_min, int e_max) {
  return amax > 0.0 ? min(e_max, max(e_min, floor_log2_d(amax) - 2)) : e_min;
}

// The softmax weights of a block's m pooling logits into w[0..m) (this wave's LDS slot):
// a_i = exp(z_i - max z) / sum_i' exp(z_i' - max z) in fp64. Ends with the slot readable.
__device__ __forceinline__ void pool_weights(const float* zb, int m, double* w) {
  const int lane = threadIdx.x & (kWave - 1);
  float zmax = -INFINITY;
  for (int i = lane; i < m; i += kWave) zmax = fmaxf(zmax, zb[i]);
  zmax = wave_max(zmax);
  double zsum = 0.0;
  for (int i = lane; i < m; i += kWave) {
    const double e = exp((double)zb[i] - (double)zmax);
    w[i] = e;
    zsum += e;
  }
  zsum = wave_sum_d(zsum);
  for (int i = lane; i < m; i += kWave) w[i] = w[i] / zsum;
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the weights are in LDS (wave-local slot)
  __builtin_amdgcn_wave_barrier();
}

// Storage of a compressed entry: bf16, e4m3fn with one fp32 scale per entry, or OCP MXFP4
// (e2m1 codes, one E8M0 exponent per 32 dims).
enum { kOutBf16 = 0, kOutFp8 = 1, kOutMxfp4 = 2 };

template <int OUT>
__global__ __launch_bounds__(kCompressWaves * kWave) void compress_kernel(
    const uint16_t* __restrict__ x, int64_t x_seq_stride, const float* __restrict__ z,
    int64_t z_seq_stride, const int64_t* __restrict__ pos0, int B, int n_ent, int D, int d_rope,
    int m, int entry_pos_offset, float rope_base, void* __restrict__ out,
    void* __restrict__ out_scale, int64_t out_seq_stride, const int32_t* __restrict__ out_entry0, float rms_eps,
    RopeTable rt) {
  __shared__ double wsh[kCompressWaves][kMaxBlock];
  const int lane = threadIdx.x & (kWave - 1);
  const int wl = threadIdx.x >> 6;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kCompressWaves + wl);
  if (w >= B * n_ent) return;
  const int b = w / n_ent;
  const int j = w - b * n_ent;
  const uint16_t* xb = x + (int64_t)b * x_seq_stride + (int64_t)j * m * D;
  const float* zb = z + (int64_t)b * z_seq_stride + (int64_t)j * m;
  double* wt = wsh[wl];

  const int cpr = D >> 3;  // 16-byte chunks per row
  const bool has0 = lane < cpr;
  const bool has1 = lane + kWave < cpr;
  // the first block of token rows is requested before the weights are formed
  uint4 v0[kUnroll], v1[kUnroll];
  auto load_block = [&](int i) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = min(i + u, m - 1);
      const uint4* row = reinterpret_cast<const uint4*>(xb + (int64_t)t * D);
      v0[u] = ld_stream16(row + (has0 ? lane : 0));
      v1[u] = ld_stream16(row + (has1 ? lane + kWave : 0));
    }
  };
  load_block(0);
  pool_weights(zb, m, wt);

  double acc0[8], acc1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc0[e] = acc1[e] = 0.0;
  // blocks of kUnroll tokens, the last one padded by repeating the final row with weight 0:
  // every load is unconditional, so a block's loads are all in flight together
  for (int i = 0; i < m; i += kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const double a = i + u < m ? wt[i + u] : 0.0;
      float f[8];
      unpack8(v0[u], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc0[e] = fma(a, (double)f[e], acc0[e]);
      unpack8(v1[u], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc1[e] = fma(a, (double)f[e], acc1[e]);
    }
    if (i + kUnroll < m) load_block(i + kUnroll);
  }
  if (!has0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc0[e] = 0.0;
  }
  if (!has1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc1[e] = 0.0;
  }

  // optional unit-gain RMSNorm of the pooled entry (before the rotation, which keeps pair norms)
  if (rms_eps > 0.f) {
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += acc0[e] * acc0[e] + acc1[e] * acc1[e];
    ss = wave_sum_d(ss);
    const double r = sqrt(ss / (double)D + (double)rms_eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc0[e] /= r;
      acc1[e] /= r;
    }
  }

  // partial RoPE on the last d_rope dims, at the entry's position (angle, sine and cosine in fp64)
  const int64_t p = pos0[b] + (int64_t)j * m + entry_pos_offset;
  const int rope0 = D - d_rope;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = lane + h * kWave;
    double* acc = h ? acc1 : acc0;
    if (c < cpr && 8 * c >= rope0) {
      const int pair0 = (8 * c - rope0) >> 1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pair = pair0 + q;
        const double ang = (double)p * (pair < kRopeTab ? rt.inv_freq[pair] : rope_inv_freq(rope_base, pair, d_rope));
        double sn, cs;
        sincos(ang, &sn, &cs);
        const double u0 = acc[2 * q], u1 = acc[2 * q + 1];
        acc[2 * q] = u0 * cs - u1 * sn;
        acc[2 * q + 1] = u0 * sn + u1 * cs;
      }
    }
  }

  const int64_t slot = (int64_t)b * out_seq_stride + (out_entry0 ? out_entry0[b] : 0) + j;
  if constexpr (OUT == kOutBf16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + slot * D;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const double* acc = h ? acc1 : acc0;
      uint4 pk;
      pk.x = f64_to_bf16_rne(acc[0]) | (f64_to_bf16_rne(acc[1]) << 16);
      pk.y = f64_to_bf16_rne(acc[2]) | (f64_to_bf16_rne(acc[3]) << 16);
      pk.z = f64_to_bf16_rne(acc[4]) | (f64_to_bf16_rne(acc[5]) << 16);
      pk.w = f64_to_bf16_rne(acc[6]) | (f64_to_bf16_rne(acc[7]) << 16);
      if (h ? has1 : has0) *reinterpret_cast<uint4*>(o + 8 * (lane + h * kWave)) = pk;
    }
  } else if constexpr (OUT == kOutFp8) {
    double amax = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmax(amax, fmax(fabs(acc0[e]), fabs(acc1[e])));
    amax = wave_max_d(amax);
    const float s = amax == 0.0 ? 1.0f : (float)(amax / 448.0);  // fp32 scale, rounded from fp64
    const double sd = (double)s;
    uint8_t* o = reinterpret_cast<uint8_t*>(out) + slot * D;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const double* acc = h ? acc1 : acc0;
      uint2 wv;
      wv.x = f64_to_e4m3(acc[0] / sd) | (f64_to_e4m3(acc[1] / sd) << 8) | (f64_to_e4m3(acc[2] / sd) << 16) |
             (f64_to_e4m3(acc[3] / sd) << 24);
      wv.y = f64_to_e4m3(acc[4] / sd) | (f64_to_e4m3(acc[5] / sd) << 8) | (f64_to_e4m3(acc[6] / sd) << 16) |
             (f64_to_e4m3(acc[7] / sd) << 24);
      if (h ? has1 : has0) *reinterpret_cast<uint2*>(o + 8 * (lane + h * kWave)) = wv;
    }
    if (lane == 0) reinterpret_cast<float*>(out_scale)[slot] = s;
  } else {
    // MXFP4: an MX block of 32 dims is 4 adjacent lanes' 8-dim chunks; E = floor(log2 amax) - 2
    // limited to the E8M0 range [-127, 127] (an all-zero block takes -127)
    uint8_t* o = reinterpret_cast<uint8_t*>(out) + slot * (D / 2);
    uint8_t* os = reinterpret_cast<uint8_t*>(out_scale) + slot * (D / 32);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = lane + h * kWave;
      const double* acc = h ? acc1 : acc0;
      double amax = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmax(amax, fabs(acc[e]));
      amax = fmax(amax, __shfl_xor(amax, 1, kWave));
      amax = fmax(amax, __shfl_xor(amax, 2, kWave));
      const int E = mx_block_exp(amax, -127, 127);
      uint32_t wv = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) wv |= e2m1_code_d(ldexp(acc[e], -E)) << (4 * e);
      if (c < cpr) {
        *reinterpret_cast<uint32_t*>(o + 4 * c) = wv;
        if ((c & 3) == 0) os[c >> 2] = (uint8_t)(E + 127);
      }
    }
  }
}

// Workgroup (b, i): token i of sequence b goes to ring slot (pos[b] + i) mod R. The position, z
// and the token's first row chunk are all requested before any is used, so the copy waits for
// one memory round trip; rows longer than 8 * blockDim.x bf16 continue in a loop.
__global__ __launch_bounds__(256) void ring_append_kernel(const uint16_t* __restrict__ x_new,
                                                          const float* __restrict__ z_new,
                                                          const int64_t* __restrict__ pos,
                                                          uint16_t* __restrict__ ring_x,
                                                          float* __restrict__ ring_z, int T, int D, int R) {
  const int b = blockIdx.x, i = blockIdx.y;
  const int64_t tok = (int64_t)b * T + i;
  const int cpr = D >> 3;
  const uint4* src = reinterpret_cast<const uint4*>(x_new + tok * D);
  const int c0 = threadIdx.x;
  const int64_t p = pos[b];
  const float z = z_new ? z_new[tok] : 0.f;
  uint4 v0 = {0u, 0u, 0u, 0u};
  if (c0 < cpr) v0 = src[c0];
  const int64_t slot = (int64_t)b * R + ((p + i) % R);
  uint4* dst = reinterpret_cast<uint4*>(ring_x + slot * D);
  if (c0 < cpr) dst[c0] = v0;
  for (int c = c0 + blockDim.x; c < cpr; c += blockDim.x) dst[c] = src[c];
  if (c0 == 0 && z_new) ring_z[slot] = z;
}

// Indexer keys of the entries: the per-token keys pooled with the entries' softmax weights (in
// fp64, like the entries), then MXFP4 (OCP MX v1.0: per 32 values E = floor(log2 amax) - 2
// within [-3, 0], elements rounded to the nearest e2m1 magnitude with ties to the even code,
// saturating at 6). One wavefront per entry; lane l holds key dims [V l, V l + V), so one MX
// block is 32 / V adjacent lanes.
constexpr int kMxEMin = -3, kMxEMax = 0;

template <int V>
__global__ __launch_bounds__(kCompressWaves * kWave) void index_key_pool_kernel(
    const uint16_t* __restrict__ xk, int64_t xk_seq_stride, const float* __restrict__ z, int64_t z_seq_stride,
    int B, int n_ent, int m, uint8_t* __restrict__ out_ik, uint8_t* __restrict__ out_iks, int64_t out_seq_stride,
    const int32_t* __restrict__ out_entry0) {
  constexpr int D_I = 64 * V;
  constexpr int LPB = 32 / V;  // lanes per MX block
  __shared__ double wsh[kCompressWaves][kMaxBlock];
  const int lane = threadIdx.x & (kWave - 1);
  const int wl = threadIdx.x >> 6;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kCompressWaves + wl);
  if (w >= B * n_ent) return;
  const int b = w / n_ent;
  const int j = w - b * n_ent;
  const uint16_t* xb = xk + (int64_t)b * xk_seq_stride + (int64_t)j * m * D_I;
  const float* zb = z + (int64_t)b * z_seq_stride + (int64_t)j * m;
  double* wt = wsh[wl];
  pool_weights(zb, m, wt);

  double acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0;
  for (int i = 0; i < m; i += kUnroll) {  // kUnroll rows in flight; the last block repeats a row with weight 0
    uint16_t r[kUnroll][V];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint16_t* row = xb + (int64_t)min(i + u, m - 1) * D_I + V * lane;
#pragma unroll
      for (int v = 0; v < V; ++v) r[u][v] = row[v];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const double a = i + u < m ? wt[i + u] : 0.0;
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = fma(a, (double)__uint_as_float((uint32_t)r[u][v] << 16), acc[v]);
    }
  }
  // block exponent
  double amax = 0.0;
#pragma unroll
  for (int v = 0; v < V; ++v) amax = fmax(amax, fabs(acc[v]));
#pragma unroll
  for (int o = 1; o < LPB; o <<= 1) amax = fmax(amax, __shfl_xor(amax, o, kWave));
  const int E = mx_block_exp(amax, kMxEMin, kMxEMax);
  uint32_t codes[V];
#pragma unroll
  for (int v = 0; v < V; ++v) codes[v] = e2m1_code_d(ldexp(acc[v], -E));
  const int64_t slot = (int64_t)b * out_seq_stride + (out_entry0 ? out_entry0[b] : 0) + j;
  uint8_t* ko = out_ik + slot * (D_I / 2);
  if constexpr (V == 1) {  // pairs of lanes form a byte
    const uint32_t hi = __shfl_down(codes[0], 1, kWave);
    if ((lane & 1) == 0) ko[lane >> 1] = (uint8_t)(codes[0] | (hi << 4));
  } else {
#pragma unroll
    for (int v = 0; v < V; v += 2) ko[(V * lane + v) >> 1] = (uint8_t)(codes[v] | (codes[v + 1] << 4));
  }
  if (lane % LPB == 0) out_iks[slot * (D_I / 32) + lane / LPB] = (uint8_t)(E + 127);
}

static int compress_impl(const char* name, const uint16_t* x, int64_t x_seq_stride, const float* z,
                         int64_t z_seq_stride, const int64_t* pos0, int B, int n_tok, int D,
                         int d_rope, int m, int entry_pos_offset, float rope_base, int out_dtype,
                         void* out, void* out_scale, int64_t out_seq_stride,
                         const int32_t* out_entry0, float rms_eps, void* stream) {
  CSKV_REQUIRE(B >= 1 && n_tok >= 0, CSKV_EINVAL, "%s: B=%d n_tok=%d", name, B, n_tok);
  CSKV_REQUIRE(m >= 1 && m <= 1024, CSKV_EINVAL, "%s: m=%d outside [1, 1024]", name, m);
  CSKV_REQUIRE(n_tok % m == 0, CSKV_EINVAL, "%s: n_tok=%d is not a multiple of m=%d", name, n_tok, m);
  CSKV_REQUIRE(D % 8 == 0 && D >= 8, CSKV_EINVAL, "%s: D=%d must be a positive multiple of 8", name, D);
  CSKV_REQUIRE(D <= 1024, CSKV_ENOTSUP, "%s: D=%d > 1024", name, D);
  CSKV_REQUIRE(d_rope >= 0 && d_rope % 8 == 0 && d_rope <= D, CSKV_EINVAL,
               "%s: d_rope=%d must be a multiple of 8 in [0, D]", name, d_rope);
  CSKV_REQUIRE(out_dtype == CSKV_BF16 || out_dtype == CSKV_FP8_E4M3 || out_dtype == CSKV_MXFP4, CSKV_EINVAL,
               "%s: unknown out_dtype %d", name, out_dtype);
  CSKV_REQUIRE(out_dtype != CSKV_MXFP4 || D % 32 == 0, CSKV_EINVAL, "%s: MXFP4 needs D %% 32 == 0 (D=%d)", name, D);
  CSKV_REQUIRE(rms_eps >= 0.f && rms_eps < INFINITY, CSKV_EINVAL, "%s: rms_eps=%g", name, (double)rms_eps);
  if (n_tok == 0) return CSKV_OK;
  CSKV_REQUIRE(x && z && pos0 && out, CSKV_EINVAL, "%s: null pointer", name);
  CSKV_REQUIRE(out_dtype == CSKV_BF16 || out_scale, CSKV_EINVAL, "%s: fp8/MXFP4 output needs out_scale", name);
  CSKV_REQUIRE(aligned16(x) && aligned16(out), CSKV_EINVAL, "%s: x/out must be 16-byte aligned", name);
  CSKV_REQUIRE(x_seq_stride % 8 == 0 && x_seq_stride >= (int64_t)n_tok * D, CSKV_EINVAL,
               "%s: x_seq_stride=%lld", name, (long long)x_seq_stride);
  CSKV_REQUIRE(z_seq_stride >= n_tok, CSKV_EINVAL, "%s: z_seq_stride=%lld", name, (long long)z_seq_stride);
  const int n_ent = n_tok / m;
  CSKV_REQUIRE(out_seq_stride >= n_ent, CSKV_EINVAL, "%s: out_seq_stride=%lld", name, (long long)out_seq_stride);
  CSKV_REQUIRE((int64_t)B * n_ent < (1ll << 31), CSKV_ENOTSUP, "%s: too many entries", name);
  const int waves = B * n_ent;
  dim3 grid((waves + kCompressWaves - 1) / kCompressWaves), block(kCompressWaves * kWave);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  RopeTable rt{};
  for (int i = 0; i < kRopeTab && i < d_rope / 2; ++i) rt.inv_freq[i] = pow((double)rope_base, -2.0 * i / d_rope);
  auto launch = [&](auto kern) {
    kern<<<grid, block, 0, s>>>(x, x_seq_stride, z, z_seq_stride, pos0, B, n_ent, D, d_rope, m, entry_pos_offset,
                                rope_base, out, out_scale, out_seq_stride, out_entry0, rms_eps, rt);
  };
  if (out_dtype == CSKV_BF16)
    launch(compress_kernel<kOutBf16>);
  else if (out_dtype == CSKV_FP8_E4M3)
    launch(compress_kernel<kOutFp8>);
  else
    launch(compress_kernel<kOutMxfp4>);
  CSKV_LAUNCH_CHECK(name);
  return CSKV_OK;
}

}  // namespace cskv

extern "C" CSKV_API int csa_compress(const uint16_t* x, int64_t x_seq_stride, const float* z,
                            int64_t z_seq_stride, const int64_t* pos0, int B, int n_tok, int D,
                            int d_rope, int m, int entry_pos_offset, float rope_base, int out_dtype,
                            void* out, void* out_scale, int64_t out_seq_stride,
                            const int32_t* out_entry0, float rms_eps, void* stream) {
  return cskv::compress_impl("csa_compress", x, x_seq_stride, z, z_seq_stride, pos0, B, n_tok, D,
                             d_rope, m, entry_pos_offset, rope_base, out_dtype, out, out_scale,
                             out_seq_stride, out_entry0, rms_eps, stream);
}

extern "C" CSKV_API int hca_compress(const uint16_t* x, int64_t x_seq_stride, const float* z,
                            int64_t z_seq_stride, const int64_t* pos0, int B, int n_tok, int D,
                            int d_rope, int m, int entry_pos_offset, float rope_base, int out_dtype,
                            void* out, void* out_scale, int64_t out_seq_stride,
                            const int32_t* out_entry0, float rms_eps, void* stream) {
  return cskv::compress_impl("hca_compress", x, x_seq_stride, z, z_seq_stride, pos0, B, n_tok, D,
                             d_rope, m, entry_pos_offset, rope_base, out_dtype, out, out_scale,
                             out_seq_stride, out_entry0, rms_eps, stream);
}

extern "C" CSKV_API int cskv_ring_append(const uint16_t* x_new, const float* z_new, const int64_t* pos,
                                uint16_t* ring_x, float* ring_z, int B, int T, int D, int R, void* stream) {
  CSKV_REQUIRE(B >= 1 && R >= 1, CSKV_EINVAL, "cskv_ring_append: B=%d R=%d", B, R);
  CSKV_REQUIRE(T >= 1 && T <= R && T <= 65535, CSKV_EINVAL, "cskv_ring_append: T=%d (ring of %d)", T, R);
  CSKV_REQUIRE(D % 8 == 0 && D >= 8, CSKV_EINVAL, "cskv_ring_append: D=%d", D);
  CSKV_REQUIRE(x_new && pos && ring_x, CSKV_EINVAL, "cskv_ring_append: null pointer");
  CSKV_REQUIRE(!z_new || ring_z, CSKV_EINVAL, "cskv_ring_append: z_new needs ring_z");
  CSKV_REQUIRE(cskv::aligned16(x_new) && cskv::aligned16(ring_x), CSKV_EINVAL,
               "cskv_ring_append: x_new/ring_x must be 16-byte aligned");
  cskv::ring_append_kernel<<<dim3(B, T), 128, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      x_new, z_new, pos, ring_x, ring_z, T, D, R);
  CSKV_LAUNCH_CHECK("cskv_ring_append");
  return CSKV_OK;
}

extern "C" CSKV_API int csa_index_key_pool(const uint16_t* xk, int64_t xk_seq_stride, const float* z,
                                           int64_t z_seq_stride, int B, int n_tok, int D_I, int m, uint8_t* out_ik,
                                           uint8_t* out_ik_scale, int64_t out_seq_stride, const int32_t* out_entry0,
                                           void* stream) {
  const char* name = "csa_index_key_pool";
  CSKV_REQUIRE(B >= 1 && n_tok >= 0, CSKV_EINVAL, "%s: B=%d n_tok=%d", name, B, n_tok);
  CSKV_REQUIRE(m >= 1 && m <= 1024, CSKV_EINVAL, "%s: m=%d outside [1, 1024]", name, m);
  CSKV_REQUIRE(n_tok % m == 0, CSKV_EINVAL, "%s: n_tok=%d is not a multiple of m=%d", name, n_tok, m);
  CSKV_REQUIRE(D_I == 64 || D_I == 128 || D_I == 256 || D_I == 512, CSKV_ENOTSUP,
               "%s: D_I=%d not in {64, 128, 256, 512}", name, D_I);
  if (n_tok == 0) return CSKV_OK;
  CSKV_REQUIRE(xk && z && out_ik && out_ik_scale, CSKV_EINVAL, "%s: null pointer", name);
  CSKV_REQUIRE(cskv::aligned16(xk), CSKV_EINVAL, "%s: xk must be 16-byte aligned", name);
  CSKV_REQUIRE(xk_seq_stride % 8 == 0 && xk_seq_stride >= (int64_t)n_tok * D_I, CSKV_EINVAL,
               "%s: xk_seq_stride=%lld", name, (long long)xk_seq_stride);
  CSKV_REQUIRE(z_seq_stride >= n_tok, CSKV_EINVAL, "%s: z_seq_stride=%lld", name, (long long)z_seq_stride);
  const int n_ent = n_tok / m;
  CSKV_REQUIRE(out_seq_stride >= n_ent, CSKV_EINVAL, "%s: out_seq_stride=%lld", name, (long long)out_seq_stride);
  CSKV_REQUIRE((int64_t)B * n_ent < (1ll << 31), CSKV_ENOTSUP, "%s: too many entries", name);
  const int waves = B * n_ent;
  dim3 grid((waves + cskv::kCompressWaves - 1) / cskv::kCompressWaves), block(cskv::kCompressWaves * cskv::kWave);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (D_I) {
    case 64:
      cskv::index_key_pool_kernel<1><<<grid, block, 0, s>>>(xk, xk_seq_stride, z, z_seq_stride, B, n_ent, m, out_ik,
                                                            out_ik_scale, out_seq_stride, out_entry0);
      break;
    case 128:
      cskv::index_key_pool_kernel<2><<<grid, block, 0, s>>>(xk, xk_seq_stride, z, z_seq_stride, B, n_ent, m, out_ik,
                                                            out_ik_scale, out_seq_stride, out_entry0);
      break;
    case 256:
      cskv::index_key_pool_kernel<4><<<grid, block, 0, s>>>(xk, xk_seq_stride, z, z_seq_stride, B, n_ent, m, out_ik,
                                                            out_ik_scale, out_seq_stride, out_entry0);
      break;
    default:
      cskv::index_key_pool_kernel<8><<<grid, block, 0, s>>>(xk, xk_seq_stride, z, z_seq_stride, B, n_ent, m, out_ik,
                                                            out_ik_scale, out_seq_stride, out_entry0);
  }
  CSKV_LAUNCH_CHECK(name);
  return CSKV_OK;
}
