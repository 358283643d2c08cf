// Shared-KV MQA attention over compressed entries plus the sliding window
// (hybrid_attn_decode, hybrid_attn_prefill).
//
// Method: page "DeepSeek-V4가 이차적 어텐션 비용 없이 백만 토큰 컨텍스트를 달성하는
// 방법", section "두 가지 압축 전략: CSA 및 HCA": CSA runs softmax attention over
// its top-k compressed entries with a sliding-window branch alongside; HCA runs
// dense attention over all of its entries; both use MQA (one KV head shared by
// all query heads) with partial RoPE. Page "딥시크 V4 분석: CSA·HCA 어텐션으로
// 100만 토큰 컨텍스트를 저비용에 구현한 방법", section "쉽게 이해하기": the window
// holds the latest 128 tokens. Entries and window tokens share one softmax.
//
// Design. One query (a decode sequence, or one prefill row) has H heads and a
// key set of compressed entries (a top-k list or a dense range) followed by
// window tokens. A workgroup takes NW waves x 16 heads and one contiguous
// split of that key set, staged 32 keys at a time into LDS as bf16 rows (fp8
// codes widen exactly; the per-entry scale is folded into the logit and into
// P; window tokens are rotated at their own position while staged). Per wave:
//   S^T-free QK: v_mfma_f32_16x16x32_bf16 with Q (rotated, in registers) as A
//               and K rows read with ds_read_b128 as B  -> S[16 heads][32 keys]
//   online softmax in the log2 domain on the accumulator lanes
//   P -> LDS as [key][head] with 8-byte writes; PV with P read back by the
//   gfx950 transposed read ds_read_b64_tr_b16 as A and V (the first d_v dims
//   of the same K rows) read by ds_read_b64_tr_b16 as B.
// Splits write unnormalised partial outputs with (max, sum) in fp32; a combine
// kernel merges them (log-sum-exp merge). One split writes the output directly.
#include <math.h>
#include <type_traits>

#include "common.cuh"
#include "host_util.h"

namespace cskv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kTK = 32;            // keys per LDS tile
constexpr int kMaxRopePairs = 64;  // d_rope <= 128
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const uint16_t* q;        // [nq, H, D]
  const int64_t* q_pos;     // [nq] (decode) or nullptr (prefill: pos0 + row)
  int64_t pos0;
  const void* ckv;          // [B_kv, N_cap, D] bf16 bits or fp8 codes
  const void* ckv_scale;    // fp32 [B_kv, N_cap] (fp8) or E8M0 bytes [B_kv, N_cap, D/32] (MXFP4)
  int kv;                   // kKvBf16, kKvFp8 or kKvMxfp4
  int N_cap;
  int64_t ckv_seq;          // entries between sequences (0: all queries share one cache)
  const int32_t* n_entries; // [nq] (decode) or nullptr (prefill: min(N, (t+1)/m))
  int m;
  const int32_t* topk;      // [nq, k] or nullptr (dense)
  int k;
  const uint16_t* win;      // decode: ring [nq, W, D]; prefill: x [T, D]
  int ring;                 // 1: slot = pos mod ring_cap, ring of sequence qi / q_per_seq; 0: row = pos - pos0 of x
  int ring_cap;             // slots per ring (>= W)
  int q_per_seq;            // consecutive queries sharing one sequence's ring and cache (decode)
  int W;
  int nq, H, D, d_rope, d_v;
  float rope_base, scale_log2;  // softmax_scale * log2(e)
  float q_rms_eps;              // > 0: unit-gain RMSNorm of each query head (folded into its logits)
  int n_splits, keys_per_split;
  uint16_t* out;            // [nq, H, d_v]
  float* out_lse;           // [nq, H]
  float* part_o;            // [nq, n_splits, H, d_v]
  float* part_ml;           // [nq, n_splits, H, 2]
  double inv_freq[kMaxRopePairs];  // RoPE frequencies base^(-2i/d_rope), formed on the host in fp64
};

// Per query: entry-key count, window start position and count.
struct KeySpace {
  int64_t t;
  int n_c;       // compressed keys (top-k slots or dense entries)
  int64_t w0;    // first window position
  int n_w;       // window tokens
};

__device__ __forceinline__ KeySpace key_space(const AttnArgs& a, int qi) {
  KeySpace ks;
  ks.t = a.q_pos ? a.q_pos[qi] : a.pos0 + qi;
  if (a.topk) {
    ks.n_c = a.k;
  } else if (a.n_entries) {
    const int n = a.n_entries[qi];
    ks.n_c = n < 0 ? 0 : (n < a.N_cap ? n : a.N_cap);
  } else {
    int64_t v = (ks.t + 1) / a.m;
    ks.n_c = (int)(v < a.N_cap ? v : a.N_cap);
  }
  const int64_t lo = a.ring ? 0 : a.pos0;
  int64_t w0 = ks.t - a.W + 1;
  if (w0 < lo) w0 = lo;
  ks.w0 = w0;
  ks.n_w = a.W > 0 ? (int)(ks.t - w0 + 1) : 0;
  return ks;
}

constexpr int kMaxSplitIdx = 1024;  // top-k slots staged per split (CSA)
constexpr float kRescaleSlack = 8.f; // log2 units the running max may run ahead of the exponent base

// LDS layout. Key rows have a pitch of D + 16 bf16 (an odd multiple of 8 dwords): the
// QK operand reads (16 rows x 16 B per lane group) and the transposed PV reads (16 rows
// x 8 B) then spread evenly over the 64 banks. P^T rows are 16 heads (8 dwords) wide.
//
// Work split. A workgroup has HG head groups of 16 heads and two waves per head group
// (2*HG waves, two per SIMD when HG = 4). Wave (hg, hf) computes S for its head group
// and keys [16hf, 16hf+16) of the 32-key tile; the two waves share the per-row maximum
// through LDS so that both use the same exponent base, each writes its half of P^T, and
// then each computes O += P V for the whole tile but only dims [hf*d_v/2, (hf+1)*d_v/2).
template <int KD, int NV, int HG>
struct AttnSmem {
  __align__(16) uint16_t kt[kTK][KD * 32 + 16];        // key rows (bf16)
  __align__(16) uint16_t pt[HG][kTK][16];              // P^T per head group: [key][head]
  __align__(16) uint16_t qr[HG * 16][kMaxRopePairs * 2 + 8];  // rotated query dims
  float xmax[2][HG][16];                               // per-half row maxima of the tile
  float kscale[kTK];              // per-key logit multiplier (log2 domain), -inf = masked
  float kvscale[kTK];             // per-key value multiplier (fp8 entry scale, else 1)
  __align__(16) float qscale[HG * 16];  // per-head logit multiplier (query RMSNorm, else 1)
  float qssr[HG * 16][kMaxRopePairs / 4];  // sum of squares of each raw rotated 8-dim query chunk
  double inv_freq[kMaxRopePairs];
  int sidx[kMaxSplitIdx];         // this split's top-k slots (CSA)
};

// Rotate 8 consecutive bf16 dims (4 RoPE pairs starting at pair0) to position pos. The angle is
// formed and reduced modulo 2*pi in fp64 (positions reach 2^20), then rotated in fp32.
__device__ __forceinline__ uint4 rope8(uint4 v, int64_t pos, const double* inv_freq, int pair0) {
  float f[8];
  unpack8(v, f);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    double ang = (double)pos * inv_freq[pair0 + p];
    ang -= 6.283185307179586476925286766559 * rint(ang * 0.15915494309189533576888376337251);
    const float af = (float)ang;  // |af| <= pi
    const float sn = __sinf(af), cs = __cosf(af);
    const float u0 = f[2 * p], u1 = f[2 * p + 1];
    f[2 * p] = u0 * cs - u1 * sn;
    f[2 * p + 1] = u0 * sn + u1 * cs;
  }
  return pack8(f);
}

// Storage of the compressed entries (ckv_dtype): bf16 rows, e4m3fn rows with one fp32 scale per
// row, or MXFP4 rows (e2m1 codes, one E8M0 exponent per 32 dims).
enum { kKvBf16 = 0, kKvFp8 = 1, kKvMxfp4 = 2 };

// One tile's raw bytes in registers: every thread's chunks are loaded with independent
// loads (issued back to back, consumed one tile later), so a tile costs one memory latency.
// A chunk is 8 dims of a bf16 row (16 bytes) or of an fp8 row (8 bytes), or one MX block of 32
// dims of an MXFP4 row (16 bytes of codes and its exponent byte).
template <int KD, int HG, int KV>
struct TileRegs {
  static constexpr int CPR = KV == kKvMxfp4 ? KD : KD * 4;  // chunks per row
  static constexpr int NT = 2 * HG * kWave;
  static constexpr int ITERS = (kTK * CPR + NT - 1) / NT;
  typename std::conditional<KV == kKvFp8, uint2, uint4>::type v[ITERS];
  uint32_t bs[KV == kKvMxfp4 ? ITERS : 1];  // MXFP4: the chunk's E8M0 byte
  float sc;
};

// Entry tiles: keys [key0, key_end) all below n_c.
template <int KD, int NV, int HG, int KV>
__device__ __forceinline__ void entry_load(const AttnArgs& a, const void* cbase, const void* sbase, int key0,
                                           int key_end, int key_begin, const AttnSmem<KD, NV, HG>& sm,
                                           TileRegs<KD, HG, KV>& R) {
  using TR = TileRegs<KD, HG, KV>;
  constexpr int D = KD * 32;
#pragma unroll
  for (int j = 0; j < TR::ITERS; ++j) {
    const int c = threadIdx.x + j * TR::NT;
    const int r = c / TR::CPR, ch = c - r * TR::CPR;
    const int key = key0 + r;
    const int idx = (c < kTK * TR::CPR && key < key_end) ? (a.topk ? sm.sidx[key - key_begin] : key) : -1;
    if constexpr (KV == kKvFp8) {
      R.v[j] = make_uint2(0, 0);
      if (idx >= 0)
        R.v[j] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(cbase) + (int64_t)idx * D + ch * 8);
    } else if constexpr (KV == kKvBf16) {
      R.v[j] = make_uint4(0, 0, 0, 0);
      if (idx >= 0)
        R.v[j] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cbase) + (int64_t)idx * D + ch * 8);
    } else {
      R.v[j] = make_uint4(0, 0, 0, 0);
      R.bs[j] = 0;
      if (idx >= 0) {
        const int64_t blk = (int64_t)idx * KD + ch;  // MX block: 16 code bytes, 1 exponent byte
        R.v[j] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(cbase) + blk * 16);
        R.bs[j] = reinterpret_cast<const uint8_t*>(sbase)[blk];
      }
    }
  }
  R.sc = -1.f;  // masked
  if (threadIdx.x < kTK) {
    const int key = key0 + threadIdx.x;
    const int idx = key < key_end ? (a.topk ? sm.sidx[key - key_begin] : key) : -1;
    if (idx >= 0) R.sc = KV == kKvFp8 ? reinterpret_cast<const float*>(sbase)[idx] : 1.f;
  }
}

template <int KD, int NV, int HG, int KV>
__device__ __forceinline__ void entry_store(const AttnArgs& a, AttnSmem<KD, NV, HG>& sm,
                                            const TileRegs<KD, HG, KV>& R) {
  using TR = TileRegs<KD, HG, KV>;
#pragma unroll
  for (int j = 0; j < TR::ITERS; ++j) {
    const int c = threadIdx.x + j * TR::NT;
    const int r = c / TR::CPR, ch = c - r * TR::CPR;
    if (c >= kTK * TR::CPR) continue;
    if constexpr (KV == kKvMxfp4) {
      // exact e2m1 * 2^E -> bf16, two values (one code byte, low nibble first) per instruction
      const float s = __builtin_amdgcn_ldexpf(1.0f, (int)R.bs[j] - 127);
      const uint32_t w[4] = {R.v[j].x, R.v[j].y, R.v[j].z, R.v[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 o;
        o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], s, 0));
        o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], s, 1));
        o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], s, 2));
        o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], s, 3));
        *reinterpret_cast<uint4*>(&sm.kt[r][32 * ch + 8 * q]) = o;
      }
      continue;
    }
    uint4 v;
    if constexpr (KV == kKvFp8) {
      // exact e4m3 -> bf16 widening, two values per instruction
      const uint32_t w0 = R.v[j].x, w1 = R.v[j].y;
      v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
      v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
      v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
      v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    } else {
      v = R.v[j];
    }
    *reinterpret_cast<uint4*>(&sm.kt[r][ch * 8]) = v;
  }
  if (threadIdx.x < kTK) {
    const float sc = R.sc;
    sm.kscale[threadIdx.x] = sc < 0.f ? -INFINITY : a.scale_log2 * sc;
    sm.kvscale[threadIdx.x] = sc < 0.f ? 0.f : sc;
  }
}

// Window tiles: keys [key0, key_end) all at or above n_c (raw bf16 tokens, rotated in LDS).
template <int KD, int NV, int HG>
__device__ __forceinline__ void window_load(const AttnArgs& a, int qi, const KeySpace& ks, int key0, int key_end,
                                            TileRegs<KD, HG, false>& R) {
  using TR = TileRegs<KD, HG, false>;
  constexpr int D = KD * 32;
#pragma unroll
  for (int j = 0; j < TR::ITERS; ++j) {
    const int c = threadIdx.x + j * TR::NT;
    const int r = c / TR::CPR, ch = c - r * TR::CPR;
    const int key = key0 + r;
    R.v[j] = make_uint4(0, 0, 0, 0);
    if (c < kTK * TR::CPR && key < key_end) {
      const int64_t pos = ks.w0 + (key - ks.n_c);
      const int64_t row = a.ring ? ((int64_t)(qi / a.q_per_seq) * a.ring_cap + pos % a.ring_cap) : (pos - a.pos0);
      R.v[j] = *reinterpret_cast<const uint4*>(a.win + row * D + ch * 8);
    }
  }
  R.sc = 0.f;
}

template <int KD, int NV, int HG>
__device__ __forceinline__ void window_store(const AttnArgs& a, const KeySpace& ks, int key0, int key_end,
                                             AttnSmem<KD, NV, HG>& sm, const TileRegs<KD, HG, false>& R) {
  using TR = TileRegs<KD, HG, false>;
  constexpr int D = KD * 32;
#pragma unroll
  for (int j = 0; j < TR::ITERS; ++j) {
    const int c = threadIdx.x + j * TR::NT;
    const int r = c / TR::CPR, ch = c - r * TR::CPR;
    if (c >= kTK * TR::CPR) continue;
    *reinterpret_cast<uint4*>(&sm.kt[r][ch * 8]) = R.v[j];
  }
  if (threadIdx.x < kTK) {
    const bool ok = key0 + (int)threadIdx.x < key_end;
    sm.kscale[threadIdx.x] = ok ? a.scale_log2 : -INFINITY;
    sm.kvscale[threadIdx.x] = ok ? 1.f : 0.f;
  }
  __syncthreads();
  // rotate the last d_rope dims in place: kTK rows x d_rope/8 chunks spread over the threads
  const int rc = a.d_rope >> 3;
  const int rope0 = D - a.d_rope;
  for (int c = threadIdx.x; c < kTK * rc; c += TR::NT) {
    const int r = c / rc, ch = c - r * rc;
    const int key = key0 + r;
    if (key < key_end) {
      uint4* p = reinterpret_cast<uint4*>(&sm.kt[r][rope0 + 8 * ch]);
      *p = rope8(*p, ks.w0 + (key - ks.n_c), sm.inv_freq, 4 * ch);
    }
  }
}

// Per-wave attention state. m is the exponent base of the running sums; it may lag the true
// running max by up to kRescaleSlack (p <= 2^8), so O is rescaled only when a logit exceeds it
// by more than that. l holds this wave's key half only; the halves are added at the end.
template <int KD, int NVH>
struct WaveState {
  uint4 qa[KD];
  f32x4 o[NVH];
  float m[4], l[4];
};

// Key row of k-slot block `half` (0: slots 0-3, 1: slots 4-7) of lane group g, lane col:
// group g's 8 k-slots are rows 4g..4g+3 and 16+4g..16+4g+3.
__device__ __forceinline__ int pv_row(int g, int col, int half) { return 16 * half + 4 * g + (col >> 2); }

// One staged tile for wave (hg, hf). Ends with the workgroup barrier that makes P^T visible.
template <int KD, int NV, int HG>
__device__ __forceinline__ void tile_compute(AttnSmem<KD, NV, HG>& sm, WaveState<KD, NV / 2>& st, int hg, int hf) {
  constexpr int NVH = NV / 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, col = lane & 15;
  const int krow = 16 * hf + col;
  // S[head 4g+r][key krow] = q_rot . k; K operands read in batches ahead of the MFMAs
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
  constexpr int BQ = 6;
#pragma unroll
  for (int s = 0; s < KD; s += BQ) {
    uint4 kv[BQ];
#pragma unroll
    for (int u = 0; u < BQ; ++u)
      if (s + u < KD) kv[u] = *reinterpret_cast<const uint4*>(&sm.kt[krow][32 * (s + u) + 8 * g]);
#pragma unroll
    for (int u = 0; u < BQ; ++u)
      if (s + u < KD)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st.qa[s + u]),
                                                       __builtin_bit_cast(bf16x8, kv[u]), sacc, 0, 0, 0);
  }
  const float ck = sm.kscale[krow], vk = sm.kvscale[krow];
  const f32x4 qs = *reinterpret_cast<const f32x4*>(&sm.qscale[16 * hg + 4 * g]);  // heads 4g..4g+3
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = ck == -INFINITY ? -INFINITY : sacc[r] * qs[r] * ck;
    const float m_ = row16_max(x[r]);
    if (col == 0) sm.xmax[hf][hg][4 * g + r] = m_;
  }
  __syncthreads();
  bool need = false;
  float mx[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mx[r] = fmaxf(sm.xmax[0][hg][4 * g + r], sm.xmax[1][hg][4 * g + r]);
    need |= mx[r] > st.m[r] + kRescaleSlack;
  }
  if (__ballot(need)) {  // rare after the first tile: move the exponent base up, rescale O and l
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mnew = mx[r] > st.m[r] + kRescaleSlack ? mx[r] : st.m[r];
      alpha[r] = st.m[r] == -INFINITY ? 0.f : exp2f(st.m[r] - mnew);
      st.l[r] *= alpha[r];
      st.m[r] = mnew;
    }
#pragma unroll
    for (int n = 0; n < NVH; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st.o[n][r] *= alpha[r];
    }
  }
  float pv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float base = st.m[r] == -INFINITY ? 0.f : st.m[r];
    const float p = exp2f(x[r] - base);
    st.l[r] += row16_sum(p);
    pv[r] = p * vk;  // value-side scale folded into P
  }
  // P^T to LDS: [key][head], 4 consecutive heads per 8-byte write
  {
    uint2 w;
    w.x = pack_bf16x2(pv[0], pv[1]);
    w.y = pack_bf16x2(pv[2], pv[3]);
    *reinterpret_cast<uint2*>(&sm.pt[hg][krow][4 * g]) = w;
  }
  __syncthreads();
  // A = P[head col][k-slots of group g] via two transposed reads of the [key][head] block
  bf16x8 pa;
  {
    const int hc = 4 * (col & 3);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(&sm.pt[hg][pv_row(g, col, 0)][hc]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(&sm.pt[hg][pv_row(g, col, 1)][hc]));
    pa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  // O[head 4g+r][dim 16(n + hf*NVH) + col] += P V over the whole tile, read in batches
  constexpr int BV = 8;
  const int r0 = pv_row(g, col, 0), r1 = pv_row(g, col, 1);
#pragma unroll
  for (int n = 0; n < NVH; n += BV) {
    i16x4 lo[BV], hi[BV];
#pragma unroll
    for (int u = 0; u < BV; ++u) {
      if (n + u < NVH) {
        const int dc = 16 * (n + u + hf * NVH) + 4 * (col & 3);
        lo[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(&sm.kt[r0][dc]));
        hi[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(&sm.kt[r1][dc]));
      }
    }
#pragma unroll
    for (int u = 0; u < BV; ++u) {
      if (n + u < NVH) {
        const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[u], hi[u], 0, 1, 2, 3, 4, 5, 6, 7));
        st.o[n + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, st.o[n + u], 0, 0, 0);
      }
    }
  }
}

template <int KD, int NV, int HG, int KV>
__global__ __launch_bounds__(2 * HG * kWave) void attn_kernel(AttnArgs a) {
  constexpr int D = KD * 32;
  constexpr int NT = 2 * HG * kWave;
  constexpr int NVH = NV / 2;
  __shared__ AttnSmem<KD, NV, HG> sm;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int hgw = wave % HG, hf = wave / HG;  // head group and key/dim half of this wave
  const int g = lane >> 4, col = lane & 15;
  const int qi = blockIdx.x;
  const int head_groups = (a.H + 16 * HG - 1) / (16 * HG);
  const int split = blockIdx.y / head_groups;
  const int wg_hg = blockIdx.y - split * head_groups;
  const int h0 = wg_hg * 16 * HG + hgw * 16;  // this wave's first head
  const int rope0 = D - a.d_rope;

  // The query loads depend on nothing else: request them first (this wave's unrotated dims into
  // its registers, this thread's first rotated chunk for the LDS copy), so that their latency
  // overlaps the position, entry-count and top-k loads below.
  const int rc = a.d_rope / 8;  // rotated 8-dim chunks per head
  WaveState<KD, NVH> st;
  {
    const int h = h0 + col;
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      const int d0 = 32 * s + 8 * g;
      st.qa[s] = make_uint4(0, 0, 0, 0);
      if (d0 < rope0 && h < a.H) st.qa[s] = *reinterpret_cast<const uint4*>(a.q + ((int64_t)qi * a.H + h) * D + d0);
    }
  }
  auto q_chunk = [&](int c) {  // raw rotated-part chunk c (head-local index c / rc) of this workgroup
    const int hl = c / rc, h = wg_hg * 16 * HG + hl;
    return h < a.H ? *reinterpret_cast<const uint4*>(a.q + ((int64_t)qi * a.H + h) * D + rope0 + 8 * (c - hl * rc))
                   : make_uint4(0, 0, 0, 0);
  };
  const uint4 qc0 = (int)threadIdx.x < HG * 16 * rc ? q_chunk(threadIdx.x) : make_uint4(0, 0, 0, 0);

  for (int i = threadIdx.x; i < a.d_rope / 2; i += NT) sm.inv_freq[i] = a.inv_freq[i];

  const KeySpace ks = key_space(a, qi);
  const int n_keys = ks.n_c + ks.n_w;
  const int key_begin = split * a.keys_per_split;
  const int key_end = min(n_keys, key_begin + a.keys_per_split);
  const int e_end = min(key_end, ks.n_c);  // entry keys [key_begin, e_end), window keys after
  if (a.topk) {
    const int n_sel = e_end - key_begin;
    for (int i = threadIdx.x; i < n_sel; i += NT) sm.sidx[i] = a.topk[(int64_t)qi * a.k + key_begin + i];
  }
  __syncthreads();  // inv_freq and sidx ready
  const bool has_e = key_begin < e_end;
  const int w_begin = max(key_begin, ks.n_c);
  const int64_t seq = (int64_t)(a.ckv_seq ? qi / a.q_per_seq : 0) * a.ckv_seq;
  constexpr int row_bytes = KV == kKvBf16 ? 2 * D : (KV == kKvFp8 ? D : D / 2);  // bytes per row: codes
  constexpr int srow_bytes = KV == kKvFp8 ? 4 : (KV == kKvMxfp4 ? D / 32 : 0);    // and scales
  const void* cbase = reinterpret_cast<const uint8_t*>(a.ckv) + seq * row_bytes;
  const void* sbase = a.ckv_scale ? reinterpret_cast<const uint8_t*>(a.ckv_scale) + seq * srow_bytes : nullptr;
  // rotated query dims -> LDS (each thread rotates whole 8-dim chunks of the WG's heads), then
  // this wave's rotated dims into its query registers; every thread calls it once
  auto rotate_query = [&]() {
    for (int c = threadIdx.x; c < HG * 16 * rc; c += NT) {
      const int hl = c / rc, ch = c - hl * rc;
      const int h = wg_hg * 16 * HG + hl;
      uint4 v = c == (int)threadIdx.x ? qc0 : q_chunk(c);
      if (h < a.H) {
        if (a.q_rms_eps > 0.f) {
          float f[8], ss = 0.f;
          unpack8(v, f);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
          sm.qssr[hl][ch] = ss;
        }
        v = rope8(v, ks.t, sm.inv_freq, 4 * ch);
      } else if (a.q_rms_eps > 0.f) {
        sm.qssr[hl][ch] = 0.f;  // padding head (no output)
      }
      *reinterpret_cast<uint4*>(&sm.qr[hl][8 * ch]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      const int d0 = 32 * s + 8 * g;
      if (d0 >= rope0) st.qa[s] = *reinterpret_cast<const uint4*>(&sm.qr[hgw * 16 + col][d0 - rope0]);
    }
  };
  // query RMSNorm: 1 / sqrt(mean(q^2) + eps) of each head over its raw D dims, applied to the
  // logits (scaling q before the product would add a bf16 rounding). The unrotated dims come
  // from this wave's query registers, the rotated ones from the chunk sums taken before the
  // rotation. Called once the first tile's loads are out, since it waits for the query loads.
  // Both waves of a head group write the same values.
  auto write_qscale = [&]() {
    float r = 1.0f;
    if (a.q_rms_eps > 0.f) {
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < KD; ++s) {
        if (32 * s + 8 * g < rope0) {
          float f[8];
          unpack8(st.qa[s], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
        }
      }
      ss += __shfl_xor(ss, 16, kWave);
      ss += __shfl_xor(ss, 32, kWave);
      for (int ch = 0; ch < a.d_rope / 8; ++ch) ss += sm.qssr[hgw * 16 + col][ch];
      r = 1.0f / sqrtf(ss / (float)D + a.q_rms_eps);
    }
    if (g == 0) sm.qscale[hgw * 16 + col] = r;
  };
#pragma unroll
  for (int n = 0; n < NVH; ++n) st.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    st.m[r] = -INFINITY;
    st.l[r] = 0.f;
  }

  TileRegs<KD, HG, false> RW;  // window tiles
  // phase 1: compressed entries. A split's first tile (entries, else window tokens) is requested
  // before the query rotation, whose arithmetic then overlaps the loads.
  if (has_e) {
    TileRegs<KD, HG, KV> R;
    entry_load<KD, NV, HG, KV>(a, cbase, sbase, key_begin, e_end, key_begin, sm, R);
    rotate_query();
    write_qscale();
    for (int key0 = key_begin; key0 < e_end; key0 += kTK) {
      __syncthreads();
      entry_store<KD, NV, HG, KV>(a, sm, R);
      __syncthreads();
      if (key0 + kTK < e_end) entry_load<KD, NV, HG, KV>(a, cbase, sbase, key0 + kTK, e_end, key_begin, sm, R);
      tile_compute<KD, NV, HG>(sm, st, hgw, hf);
    }
  } else {
    if (w_begin < key_end) window_load<KD, NV, HG>(a, qi, ks, w_begin, key_end, RW);
    rotate_query();
  }
  // phase 2: window tokens
  if (w_begin < key_end) {
    if (has_e)
      window_load<KD, NV, HG>(a, qi, ks, w_begin, key_end, RW);
    else
      write_qscale();
    for (int key0 = w_begin; key0 < key_end; key0 += kTK) {
      __syncthreads();
      window_store<KD, NV, HG>(a, ks, key0, key_end, sm, RW);
      __syncthreads();
      if (key0 + kTK < key_end) window_load<KD, NV, HG>(a, qi, ks, key0 + kTK, key_end, RW);
      tile_compute<KD, NV, HG>(sm, st, hgw, hf);
    }
  }

  // combine the two key halves' sums: l = l_0 + l_1 (same exponent base m)
  __syncthreads();
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.xmax[hf][hgw][4 * g + r] = st.l[r];
  }
  __syncthreads();
  float lt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lt[r] = sm.xmax[0][hgw][4 * g + r] + sm.xmax[1][hgw][4 * g + r];

  // write: direct (one split) or partial; this wave owns dims [hf*d_v/2, (hf+1)*d_v/2)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = h0 + 4 * g + r;
    if (h >= a.H) continue;
    if (a.n_splits == 1) {
      const float inv = lt[r] > 0.f ? 1.f / lt[r] : 0.f;
      uint16_t* dst = a.out + ((int64_t)qi * a.H + h) * a.d_v + hf * 16 * NVH;
#pragma unroll
      for (int n = 0; n < NVH; ++n) dst[16 * n + col] = (uint16_t)f32_to_bf16_rne(st.o[n][r] * inv);
      if (a.out_lse && col == 0 && hf == 0)
        a.out_lse[(int64_t)qi * a.H + h] = lt[r] > 0.f ? (st.m[r] + log2f(lt[r])) * kLn2 : -INFINITY;
    } else {
      const int64_t pidx = ((int64_t)qi * a.n_splits + split) * a.H + h;
      float* dst = a.part_o + pidx * a.d_v + hf * 16 * NVH;
#pragma unroll
      for (int n = 0; n < NVH; ++n) dst[16 * n + col] = st.o[n][r];
      if (col == 0 && hf == 0) {
        a.part_ml[pidx * 2 + 0] = st.m[r];
        a.part_ml[pidx * 2 + 1] = lt[r];
      }
    }
  }
}

// One workgroup per (query, head): log-sum-exp merge of the split partials. Thread t owns
// dims 4t..4t+3 (d_v <= 4 * kCombNT). Split rows are read in batches of kCombBatch into two
// alternating register buffers, each batch requested before the previous one is summed; the
// first batch and every split's (m, l) are requested together, so the weights are formed while
// the first rows are in flight. The split count is padded to a whole batch with rows clamped to
// the last split and zero weights, so every load of a batch is unconditional; each exit of the
// loop sums its last batch itself, so no fetch is ever left unused (which would let the
// compiler move it behind the exit) and the waits stay exact.
constexpr int kMaxSplits = 256;
constexpr int kCombNT = 128;
constexpr int kCombBatch = 8;
__global__ __launch_bounds__(kCombNT) void attn_combine_kernel(AttnArgs a) {
  __shared__ float wsh[kMaxSplits + 2 * kCombBatch];
  __shared__ float red[2][2];
  const int qi = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int S = a.n_splits, SP = (S + kCombBatch - 1) / kCombBatch * kCombBatch;
  const int lane = tid & (kWave - 1), w = tid >> 6;
  const int64_t base = (int64_t)qi * S, srow = (int64_t)a.H * a.d_v;
  const int dd = min(4 * tid, a.d_v - 4);  // threads past d_v read the last dims and store nothing
  const float* po = a.part_o + (base * a.H + h) * a.d_v + dd;  // split s at po[s * srow]
  const float2* pml = reinterpret_cast<const float2*>(a.part_ml) + base * a.H + h;  // split s at pml[s * H]
  float2 ml[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) ml[j] = pml[min(tid + j * kCombNT, S - 1) * a.H];
  f32x4 v0[kCombBatch], v1[kCombBatch];
#pragma unroll
  for (int u = 0; u < kCombBatch; ++u) v0[u] = *reinterpret_cast<const f32x4*>(po + min(u, S - 1) * srow);
  float mloc = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (tid + j * kCombNT < S) mloc = fmaxf(mloc, ml[j].x);
  mloc = wave_max(mloc);
  if (lane == 0) red[0][w] = mloc;
  __syncthreads();
  const float M = fmaxf(red[0][0], red[0][1]);
  const float Mb = M == -INFINITY ? 0.f : M;
  float lloc = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sp = tid + j * kCombNT;
    if (sp < S) {
      const float wt = exp2f(ml[j].x - Mb);
      wsh[sp] = wt;
      lloc += wt * ml[j].y;
    } else if (sp < SP) {
      wsh[sp] = 0.f;
    }
  }
  lloc = wave_sum(lloc);
  if (lane == 0) red[1][w] = lloc;
  __syncthreads();
  const float L = red[1][0] + red[1][1];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto fetch = [&](f32x4 (&v)[kCombBatch], int s0) {
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) v[u] = *reinterpret_cast<const f32x4*>(po + min(s0 + u, S - 1) * srow);
  };
  auto sum = [&](const f32x4 (&v)[kCombBatch], int s0) {
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) {
      const float wt = wsh[s0 + u];
      acc.x += wt * v[u].x;
      acc.y += wt * v[u].y;
      acc.z += wt * v[u].z;
      acc.w += wt * v[u].w;
    }
  };
  for (int s0 = 0;; s0 += 2 * kCombBatch) {  // v0 holds rows s0.. on entry
    if (s0 + kCombBatch >= SP) {  // v0 is the last batch
      sum(v0, s0);
      break;
    }
    fetch(v1, s0 + kCombBatch);
    sum(v0, s0);
    if (s0 + 2 * kCombBatch >= SP) {  // v1 is the last batch
      sum(v1, s0 + kCombBatch);
      break;
    }
    fetch(v0, s0 + 2 * kCombBatch);
    sum(v1, s0 + kCombBatch);
  }
  if (4 * tid < a.d_v) {
    uint2 packed;
    packed.x = pack_bf16x2(acc.x * inv, acc.y * inv);
    packed.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(a.out + ((int64_t)qi * a.H + h) * a.d_v + dd) = packed;
  }
  if (tid == 0 && a.out_lse)
    a.out_lse[(int64_t)qi * a.H + h] = L > 0.f ? (Mb + log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- host side
struct AttnPlan {
  int nw, n_splits, keys_per_split;
  size_t ws;
};

static AttnPlan plan_attn(int nq, int H, int d_v, int max_keys) {
  AttnPlan p;
  p.nw = H >= 64 ? 4 : (H + 15) / 16;  // head groups of 16 per workgroup (two waves each)
  const int head_groups = (H + 16 * p.nw - 1) / (16 * p.nw);
  const int64_t base = (int64_t)nq * head_groups;
  // one workgroup per CU (256) when the queries alone do not fill the GPU; a split holds at
  // least one tile and at most kMaxSplitIdx keys, and there are at most kMaxSplits splits
  int splits = (int)((256 + base - 1) / base);
  const int max_splits = (max_keys + kTK - 1) / kTK;
  if (splits > max_splits) splits = max_splits;
  const int min_splits = (max_keys + kMaxSplitIdx - 1) / kMaxSplitIdx;
  if (splits < min_splits) splits = min_splits;
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits < 1) splits = 1;
  int per = (max_keys + splits - 1) / splits;
  per = (per + kTK - 1) / kTK * kTK;
  if (per < kTK) per = kTK;
  if (per > kMaxSplitIdx) per = kMaxSplitIdx;
  splits = (max_keys + per - 1) / per;
  if (splits < 1) splits = 1;
  p.n_splits = splits;
  p.keys_per_split = per;
  p.ws = splits > 1 ? (size_t)nq * splits * H * (d_v + 2) * sizeof(float) : 0;
  return p;
}

typedef void (*AttnKernel)(AttnArgs);

template <int KD, int NV, int KV>
static AttnKernel pick_nw(int hg) {
  switch (hg) {
    case 1: return attn_kernel<KD, NV, 1, KV>;
    case 2: return attn_kernel<KD, NV, 2, KV>;
    case 3: return attn_kernel<KD, NV, 3, KV>;
    default: return attn_kernel<KD, NV, 4, KV>;
  }
}

template <int KV>
static AttnKernel pick_dims(int D, int d_v, int nw) {
  if (D == 576 && d_v == 512) return pick_nw<18, 32, KV>(nw);
  if (D == 128 && d_v == 128) return pick_nw<4, 8, KV>(nw);
  if (D == 64 && d_v == 32) return pick_nw<2, 2, KV>(nw);
  if (D == 256 && d_v == 128) return pick_nw<8, 8, KV>(nw);
  return nullptr;
}

// Compiled (D, d_v) pairs.
static AttnKernel pick_kernel(int D, int d_v, int nw, int kv) {
  return kv == kKvFp8 ? pick_dims<kKvFp8>(D, d_v, nw)
                      : (kv == kKvMxfp4 ? pick_dims<kKvMxfp4>(D, d_v, nw) : pick_dims<kKvBf16>(D, d_v, nw));
}

static int check_common(const char* name, int H, int D, int d_rope, int d_v, int W, int ckv_dtype, float q_rms_eps) {
  CSKV_REQUIRE(H >= 1 && H <= 128, CSKV_EINVAL, "%s: H=%d outside [1, 128]", name, H);
  CSKV_REQUIRE(D % 32 == 0 && D >= 32, CSKV_EINVAL, "%s: D=%d must be a positive multiple of 32", name, D);
  CSKV_REQUIRE(d_v % 16 == 0 && d_v >= 16 && d_v <= D, CSKV_EINVAL, "%s: d_v=%d", name, d_v);
  CSKV_REQUIRE(d_rope >= 0 && d_rope % 8 == 0 && d_rope <= D, CSKV_EINVAL, "%s: d_rope=%d", name, d_rope);
  CSKV_REQUIRE(W >= 0, CSKV_EINVAL, "%s: W=%d", name, W);
  CSKV_REQUIRE(q_rms_eps >= 0.f && q_rms_eps < INFINITY, CSKV_EINVAL, "%s: q_rms_eps=%g", name, (double)q_rms_eps);
  CSKV_REQUIRE(d_rope <= 2 * kMaxRopePairs, CSKV_ENOTSUP, "%s: d_rope=%d > %d", name, d_rope, 2 * kMaxRopePairs);
  CSKV_REQUIRE(ckv_dtype == CSKV_BF16 || ckv_dtype == CSKV_FP8_E4M3 || ckv_dtype == CSKV_MXFP4, CSKV_EINVAL,
               "%s: ckv_dtype=%d", name, ckv_dtype);
  CSKV_REQUIRE(d_v % 32 == 0, CSKV_ENOTSUP, "%s: d_v=%d must be a multiple of 32", name, d_v);
  CSKV_REQUIRE(pick_kernel(D, d_v, 1, kKvBf16) != nullptr, CSKV_ENOTSUP,
               "%s: (D, d_v) = (%d, %d) not compiled (576/512, 128/128, 256/128, 64/32)", name, D, d_v);
  return CSKV_OK;
}

static int launch_attn(const char* name, AttnArgs a, const AttnPlan& p, void* ws, size_t ws_bytes, hipStream_t s) {
  for (int i = 0; i < a.d_rope / 2; ++i) a.inv_freq[i] = pow((double)a.rope_base, -2.0 * (double)i / (double)a.d_rope);
  CSKV_REQUIRE(p.ws == 0 || (ws && ws_bytes >= p.ws), CSKV_EWORKSPACE, "%s: workspace %zu < %zu bytes", name,
               ws_bytes, p.ws);
  CSKV_REQUIRE(p.n_splits == 1 || a.d_v <= 4 * kCombNT, CSKV_ENOTSUP, "%s: d_v=%d > %d with split keys", name,
               a.d_v, 4 * kCombNT);
  a.n_splits = p.n_splits;
  a.keys_per_split = p.keys_per_split;
  if (p.n_splits > 1) {
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = a.part_o + (size_t)a.nq * p.n_splits * a.H * a.d_v;
  }
  const int head_groups = (a.H + 16 * p.nw - 1) / (16 * p.nw);
  AttnKernel kern = pick_kernel(a.D, a.d_v, p.nw, a.kv);
  hipLaunchKernelGGL(kern, dim3(a.nq, p.n_splits * head_groups), dim3(2 * p.nw * kWave), 0, s, a);
  CSKV_LAUNCH_CHECK(name);
  if (p.n_splits > 1) {
    hipLaunchKernelGGL(attn_combine_kernel, dim3(a.nq, a.H), dim3(kCombNT), 0, s, a);
    CSKV_LAUNCH_CHECK(name);
  }
  return CSKV_OK;
}

}  // namespace cskv

using namespace cskv;

extern "C" CSKV_API size_t hybrid_attn_decode_workspace_size(int B, int H, int d_v, int N_cap, int k, int W, int dense) {
  if (B < 1 || H < 1 || d_v < 1) return 0;
  const int max_keys = (dense ? N_cap : k) + (W > 0 ? W : 0);
  return plan_attn(B, H, d_v, max_keys > 0 ? max_keys : 1).ws;
}

extern "C" CSKV_API int hybrid_attn_decode(const uint16_t* q, const int64_t* q_pos, const void* ckv,
                                           const void* ckv_scale, int ckv_dtype, int N_cap,
                                           const int32_t* n_entries, const int32_t* topk_idx, int k,
                                           const uint16_t* win, int W, int B, int H, int D, int d_rope, int d_v,
                                           float rope_base, float softmax_scale, uint16_t* out, float* out_lse,
                                           void* ws, size_t ws_bytes, float q_rms_eps, int T, int R,
                                           void* stream) {
  const char* name = "hybrid_attn_decode";
  CSKV_REQUIRE(B >= 1 && N_cap >= 0, CSKV_EINVAL, "%s: B=%d N_cap=%d", name, B, N_cap);
  if (R == 0) R = W;
  CSKV_REQUIRE(T >= 1 && (int64_t)B * T < (1 << 20), CSKV_EINVAL, "%s: T=%d", name, T);
  CSKV_REQUIRE(W == 0 || R >= W, CSKV_EINVAL, "%s: ring of %d slots < window %d", name, R, W);
  int rc = check_common(name, H, D, d_rope, d_v, W, ckv_dtype, q_rms_eps);
  if (rc) return rc;
  CSKV_REQUIRE(!topk_idx || k >= 1, CSKV_EINVAL, "%s: k=%d", name, k);
  CSKV_REQUIRE(q && q_pos && out && n_entries, CSKV_EINVAL, "%s: null pointer", name);
  CSKV_REQUIRE(W == 0 || win, CSKV_EINVAL, "%s: null window", name);
  CSKV_REQUIRE(N_cap == 0 || (ckv && (ckv_dtype == CSKV_BF16 || ckv_scale)), CSKV_EINVAL, "%s: null cache", name);
  CSKV_REQUIRE(aligned16(q) && aligned16(ckv) && aligned16(win), CSKV_EINVAL, "%s: q/ckv/win must be 16-byte aligned",
               name);
  const int max_keys = (topk_idx ? k : N_cap) + W;
  AttnPlan p = plan_attn(B * T, H, d_v, max_keys > 0 ? max_keys : 1);
  AttnArgs a{};
  a.q = q;
  a.q_pos = q_pos;
  a.pos0 = 0;
  a.ckv = ckv;
  a.ckv_scale = ckv_scale;
  a.kv = ckv_dtype == CSKV_FP8_E4M3 ? kKvFp8 : (ckv_dtype == CSKV_MXFP4 ? kKvMxfp4 : kKvBf16);
  a.N_cap = N_cap;
  a.ckv_seq = N_cap;
  a.n_entries = n_entries;
  a.m = 1;
  a.topk = topk_idx;
  a.k = k;
  a.win = win;
  a.ring = 1;
  a.ring_cap = R;
  a.q_per_seq = T;
  a.W = W;
  a.nq = B * T;
  a.H = H;
  a.D = D;
  a.d_rope = d_rope;
  a.d_v = d_v;
  a.rope_base = rope_base;
  a.scale_log2 = softmax_scale * kLog2e;
  a.q_rms_eps = q_rms_eps;
  a.out = out;
  a.out_lse = out_lse;
  return launch_attn(name, a, p, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

extern "C" CSKV_API size_t hybrid_attn_prefill_workspace_size(int T, int H, int d_v, int N, int k, int W, int dense) {
  return hybrid_attn_decode_workspace_size(T, H, d_v, N, k, W, dense);
}

extern "C" CSKV_API int hybrid_attn_prefill(const uint16_t* q, int64_t pos0, int T, const void* ckv,
                                            const void* ckv_scale, int ckv_dtype, int N, const int32_t* topk_idx,
                                            int k, const uint16_t* x, int W, int H, int D, int d_rope, int d_v,
                                            int m, float rope_base, float softmax_scale, uint16_t* out,
                                            float* out_lse, void* ws, size_t ws_bytes, float q_rms_eps,
                                            void* stream) {
  const char* name = "hybrid_attn_prefill";
  CSKV_REQUIRE(T >= 0 && N >= 0 && pos0 >= 0 && m >= 1, CSKV_EINVAL, "%s: T=%d N=%d pos0=%lld m=%d", name, T, N,
               (long long)pos0, m);
  int rc = check_common(name, H, D, d_rope, d_v, W, ckv_dtype, q_rms_eps);
  if (rc) return rc;
  if (T == 0) return CSKV_OK;
  CSKV_REQUIRE(!topk_idx || k >= 1, CSKV_EINVAL, "%s: k=%d", name, k);
  CSKV_REQUIRE(q && out && (W == 0 || x), CSKV_EINVAL, "%s: null pointer", name);
  CSKV_REQUIRE(N == 0 || (ckv && (ckv_dtype == CSKV_BF16 || ckv_scale)), CSKV_EINVAL, "%s: null cache", name);
  CSKV_REQUIRE(aligned16(q) && aligned16(ckv) && aligned16(x), CSKV_EINVAL, "%s: q/ckv/x must be 16-byte aligned",
               name);
  const int max_keys = (topk_idx ? k : N) + W;
  AttnPlan p = plan_attn(T, H, d_v, max_keys > 0 ? max_keys : 1);
  AttnArgs a{};
  a.q = q;
  a.q_pos = nullptr;
  a.pos0 = pos0;
  a.ckv = ckv;
  a.ckv_scale = ckv_scale;
  a.kv = ckv_dtype == CSKV_FP8_E4M3 ? kKvFp8 : (ckv_dtype == CSKV_MXFP4 ? kKvMxfp4 : kKvBf16);
  a.N_cap = N;
  a.ckv_seq = 0;
  a.n_entries = nullptr;
  a.m = m;
  a.topk = topk_idx;
  a.k = k;
  a.win = x;
  a.ring = 0;
  a.ring_cap = W;
  a.q_per_seq = 1;
  a.W = W;
  a.nq = T;
  a.H = H;
  a.D = D;
  a.d_rope = d_rope;
  a.d_v = d_v;
  a.rope_base = rope_base;
  a.scale_log2 = softmax_scale * kLog2e;
  a.q_rms_eps = q_rms_eps;
  a.out = out;
  a.out_lse = out_lse;
  return launch_attn(name, a, p, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}
