// Shared-KV MQA attention over compressed entries plus the sliding window: the kernel for short
// key sets (a few hundred keys per query, few queries), the workgroup holding 16 heads.
//
// Method: page "DeepSeek-V4가 이차적 어텐션 비용 없이 백만 토큰 컨텍스트를 달성하는
// 방법", section "두 가지 압축 전략: CSA 및 HCA" (CSA: softmax attention over the top-k
// compressed entries with a sliding-window branch; HCA: dense over all entries; MQA with partial
// RoPE); page "딥시크 V4 분석: CSA·HCA 어텐션으로 100만 토큰 컨텍스트를 저비용에 구현한
// 방법", section "쉽게 이해하기" (the window holds the latest 128 tokens).
//
// Design. A workgroup of four waves takes one query, one group of 16 heads (the 16 rows of a
// v_mfma_f32_16x16x32_bf16) and one split of the key set; two workgroups share a CU, so one
// workgroup's row lookups and first loads overlap the other's tiles, which is what a key set of
// a few tiles needs. Keys are staged through LDS a tile at a time, the next tile's rows
// travelling in registers: fp8 entries as 64-key tiles of codes widened to bf16 as they are read,
// bf16 and MXFP4 entries and window tokens as 32-key bf16 tiles (window tokens rotated at their own
// position while staged). Per tile, wave w computes S = Q K^T for keys [16w, 16w+16) with the
// rotated query in registers; the tile's per-head maxima meet in LDS; the online softmax runs in
// the log2 domain; P^T goes to LDS as [key][head]; wave w computes O += P V for a quarter of the
// value dims, reading P and V with the transposed LDS reads ds_read_b64_tr_b16 / _tr_b8. The
// rotated dims of the query and of window keys go through the MFMA as a bf16 value plus a bf16
// remainder. A query's splits write unnormalised partials merged by a second launch.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "common.cuh"
#include "host_util.h"
#include "attention_call.h"

namespace cskv {
namespace g16 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kNT = 256;             // threads per workgroup (4 waves)
constexpr int kHG = 16;              // heads per workgroup
constexpr int kTK8 = 64;             // keys per fp8 entry tile
constexpr int kTK16 = 32;            // keys per bf16 tile
constexpr int kRB = 2;               // 32-dim blocks holding rotated dims (d_rope <= 64)
constexpr int kMaxRopePairs = 32;
constexpr int kMaxSplitKeys = 4096;  // key rows staged per split
constexpr int kMaxSplits = 64;
constexpr int kTargetWG = 512;      // workgroups a launch aims at (two per CU)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;  // log2 units the running max may run ahead of the exponent base


struct AttnArgs {
  const uint16_t* q;         // [nq, H, D]
  const int64_t* q_pos;      // [nq] (decode) or nullptr (prefill: pos0 + row)
  int64_t pos0;
  const void* ckv;           // [B_kv, N_cap, D] bf16 bits, fp8 codes, or MXFP4 codes [.., D/2]
  const void* ckv_scale;     // fp32 [B_kv, N_cap] (fp8) or E8M0 bytes [B_kv, N_cap, D/32] (MXFP4)
  int kv_dtype;              // kKvBf16, kKvFp8 or kKvMxfp4
  int N_cap;
  int64_t ckv_seq;           // entries between sequences (0: all queries share one cache)
  const int32_t* n_entries;  // [nq] (decode) or nullptr (prefill: min(N, (t+1)/m))
  int m;
  const int32_t* topk;       // [nq, k] or nullptr (dense)
  int k;
  const uint16_t* win;       // decode: rings [B, R, D]; prefill: x [T, D]
  int ring;                  // 1: slot = pos mod ring_cap of sequence qi / q_per_seq; 0: row = pos - pos0 of x
  int ring_cap;
  int q_per_seq;             // consecutive queries sharing one sequence's ring and cache (decode)
  int W;
  int nq, H, D, d_rope, d_v;
  float rope_base;
  float scale_log2;          // softmax_scale * log2(e)
  float q_rms_eps;           // > 0: unit-gain RMSNorm of each query head (folded into its logits)
  int n_hg;                  // head groups of 16
  int n_splits, keys_per_split;
  int xcd_map;               // 1: a query's workgroups are issued to one XCD (round-robin dispatch)
  uint16_t* out;             // [nq, H, d_v]
  float* out_lse;            // [nq, H]
  float* part_o;             // [nq, n_hg, n_splits, 16, d_v]
  float* part_ml;            // [nq, n_hg, n_splits, 16, 2]
  const uint16_t* x_new;     // append mode: [B, T, D] new tokens (rows >= kNewRow), else nullptr
  const float* z_new;        // [B, T] or nullptr
  uint16_t* ring_w;          // the rings (win), written in append mode
  float* ring_z;             // [B, R] (with z_new)
  double rev_freq[kMaxRopePairs];  // RoPE frequencies base^(-2i/d_rope) / (2 pi), formed on the host in fp64
};

// Per query: entry-key count, window start position and count.
struct KeySpace {
  int64_t t;
  int n_c;     // compressed keys (top-k slots or dense entries)
  int64_t w0;  // first window position
  int n_w;     // window tokens
};

__device__ __forceinline__ KeySpace key_space(const AttnArgs& a, int qi) {
  KeySpace ks;
  ks.t = a.q_pos ? a.q_pos[qi] : a.pos0 + qi;
  if (a.N_cap == 0) {
    ks.n_c = 0;  // no cache (every top-k slot would be masked)
  } else if (a.topk) {
    ks.n_c = a.k;
  } else if (a.n_entries) {
    const int n = a.n_entries[qi];
    ks.n_c = n < 0 ? 0 : (n < a.N_cap ? n : a.N_cap);
  } else {
    const int64_t v = (ks.t + 1) / a.m;
    ks.n_c = (int)(v < a.N_cap ? v : a.N_cap);
  }
  const int64_t lo = a.ring ? 0 : a.pos0;
  int64_t w0 = ks.t - a.W + 1;
  if (w0 < lo) w0 = lo;
  ks.w0 = w0;
  ks.n_w = a.W > 0 ? (int)(ks.t - w0 + 1) : 0;
  return ks;
}

// cos / sin of the RoPE angle pos * inv_freq, with rev = inv_freq / (2 pi) (host fp64): the angle
// in revolutions is formed and reduced to [-1/2, 1/2] in fp64 (positions reach 2^20), then
// evaluated with the hardware sine and cosine, which take revolutions (error of order 2^-22).
__device__ __forceinline__ void rope_cs(double rev, int64_t pos, float* c, float* s) {
  double r = (double)pos * rev;
  r -= rint(r);
  const float rf = (float)r;
  *s = __builtin_amdgcn_sinf(rf);
  *c = __builtin_amdgcn_cosf(rf);
}

// Rotates 8 consecutive bf16 dims (RoPE pairs pair0 .. pair0 + 3) to position pos in fp32 and
// returns the rotated values as bf16 (hi) and the bf16 rounding of the remainder (lo).
__device__ __forceinline__ void rope8_hi_lo(uint4 v, int64_t pos, const double* rev, int pair0, uint4* hi,
                                           uint4* lo) {
  float f[8];
  unpack8(v, f);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float cs, sn;
    rope_cs(rev[pair0 + p], pos, &cs, &sn);
    const float u0 = f[2 * p], u1 = f[2 * p + 1];
    f[2 * p] = u0 * cs - u1 * sn;
    f[2 * p + 1] = u0 * sn + u1 * cs;
  }
  const uint4 h = pack8(f);
  float hf[8], r[8];
  unpack8(h, hf);
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = f[e] - hf[e];
  *hi = h;
  *lo = pack8(r);
}

// Eight e4m3 codes (two dwords, element i in byte i) -> eight bf16 (exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  uint4 v;
  v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(bf16x8, v);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// LDS. Tiles: fp8 rows of D + 16 bytes, bf16 rows of D + 16 elements (both keep the MFMA operand
// reads and the transposed reads free of bank conflicts), window remainders of the rotated
// 32-dim blocks in klo. P^T is [key][head].
template <int KD>
struct AttnSmem {
  union {
    __align__(16) uint8_t k8[kTK8][KD * 32 + 16];
    struct {
      __align__(16) uint16_t k16[kTK16][KD * 32 + 16];
      __align__(16) uint16_t klo[kTK16][kRB * 32 + 8];
    } b;
  } t;
  __align__(16) uint16_t pt[kTK8][kHG];
  float xmax[4][kHG];
  float lsum[4][kHG];
  float kscale[kTK8];   // per-key logit multiplier (log2 domain), -inf = masked
  float kvscale[kTK8];  // per-key value multiplier (fp8 entry scale, else 1), 0 = masked
  __align__(16) float qscale[kHG];
  __align__(16) uint16_t qrh[kHG][2 * kMaxRopePairs];  // rotated query dims: bf16 value
  __align__(16) uint16_t qrl[kHG][2 * kMaxRopePairs];  // and bf16 remainder
  int sidx[kMaxSplitKeys];
};

// One tile's raw rows in registers. Thread t owns row t / TPR of the tile and its 16-byte chunks
// t % TPR + TPR i (an MX block of 32 dims with its exponent byte for MXFP4), so it looks its row
// up once and issues its loads from one base address. In a window row, thread j of the row also
// owns the row's rotated chunk j (d_rope <= 64: at most 8 of them). Entry tiles and window tiles
// share the registers (the first window tile is requested while the last entry tile is computed).
template <int KD, int KV>
struct EntryGeom {
  static constexpr int TK = KV == kKvFp8 ? kTK8 : kTK16;
  static constexpr int TPR = kNT / TK;  // threads per row
  static constexpr int CPR = KV == kKvFp8 ? KD * 2 : (KV == kKvBf16 ? KD * 4 : KD);  // chunks per row
  static constexpr int NC = (CPR + TPR - 1) / TPR;  // chunks per thread
};
template <int KD>
struct WinGeom {
  static constexpr int TPR = kNT / kTK16;
  static constexpr int CPR = KD * 4;
  static constexpr int NC = (CPR + TPR - 1) / TPR;
};
template <int KD, int KV>
struct TileRegs {
  static constexpr int NV = EntryGeom<KD, KV>::NC > WinGeom<KD>::NC ? EntryGeom<KD, KV>::NC : WinGeom<KD>::NC;
  uint4 v[NV];
  uint4 rot;  // window tiles: this thread's rotated chunk
  uint32_t bs[KV == kKvMxfp4 ? EntryGeom<KD, KV>::NC : 1];
  float sc;
  int row;    // -1: masked
};

// Tile loads. The rows of a split's keys were resolved into sm.sidx (entry row in the cache,
// window row in win, -1 = masked). Loads are unconditional (a masked row reads row 0, a chunk past
// the row end its last chunk); the store writes zeros for a masked row (a masked key gets p = 0,
// which must not meet a non-finite value in the MFMA).
template <int KD, int KV>
__device__ __forceinline__ void entry_load(const uint8_t* cbase, const uint8_t* sbase, int key0, int key_end,
                                           int key_begin, const AttnSmem<KD>& sm, TileRegs<KD, KV>& R) {
  using EG = EntryGeom<KD, KV>;
  constexpr int D = KD * 32;
  constexpr int RB = KV == kKvBf16 ? 2 * D : (KV == kKvFp8 ? D : D / 2);  // code bytes per row
  const int r = threadIdx.x / EG::TPR, c0 = threadIdx.x % EG::TPR;
  const int row = key0 + r < key_end ? sm.sidx[key0 - key_begin + r] : -1;
  R.row = row;
  const int64_t rr = max(row, 0);
  const uint8_t* src = cbase + rr * RB;
#pragma unroll
  for (int i = 0; i < EG::NC; ++i) {
    const int ch = EG::CPR % EG::TPR == 0 ? c0 + EG::TPR * i : min(c0 + EG::TPR * i, EG::CPR - 1);
    R.v[i] = *reinterpret_cast<const uint4*>(src + 16 * ch);
    if constexpr (KV == kKvMxfp4) R.bs[i] = sbase[rr * KD + ch];
  }
  R.sc = KV == kKvFp8 ? reinterpret_cast<const float*>(sbase)[rr] : 1.f;
}

template <int KD, int KV>
__device__ __forceinline__ void entry_store(const AttnArgs& a, AttnSmem<KD>& sm, const TileRegs<KD, KV>& R) {
  using EG = EntryGeom<KD, KV>;
  const int r = threadIdx.x / EG::TPR, c0 = threadIdx.x % EG::TPR;
  const bool ok = R.row >= 0;
#pragma unroll
  for (int i = 0; i < EG::NC; ++i) {
    const int ch = c0 + EG::TPR * i;
    if (EG::CPR % EG::TPR != 0 && ch >= EG::CPR) continue;
    if constexpr (KV == kKvFp8) {
      *reinterpret_cast<uint4*>(&sm.t.k8[r][16 * ch]) = ok ? R.v[i] : make_uint4(0, 0, 0, 0);
    } else if constexpr (KV == kKvBf16) {
      *reinterpret_cast<uint4*>(&sm.t.b.k16[r][8 * ch]) = ok ? R.v[i] : make_uint4(0, 0, 0, 0);
    } else {
      // exact e2m1 * 2^E -> bf16, two values (one code byte, low nibble first) per instruction
      const float s = __builtin_amdgcn_ldexpf(1.0f, (int)R.bs[i] - 127);
      const uint32_t wd[4] = {R.v[i].x, R.v[i].y, R.v[i].z, R.v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 o;
        o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[q], s, 0));
        o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[q], s, 1));
        o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[q], s, 2));
        o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[q], s, 3));
        *reinterpret_cast<uint4*>(&sm.t.b.k16[r][32 * ch + 8 * q]) = ok ? o : make_uint4(0, 0, 0, 0);
      }
    }
  }
  if (c0 == 0) {
    sm.kscale[r] = ok ? a.scale_log2 * R.sc : -INFINITY;
    sm.kvscale[r] = ok ? R.sc : 0.f;
  }
}

// Window rows: thread j of a row takes its unrotated chunks j + 8 i and, for j < d_rope/8, the
// rotated chunk j.
template <int KD, int KV>
__device__ __forceinline__ void window_load(const AttnArgs& a, int key0, int key_end, int key_begin, int rope0,
                                            const AttnSmem<KD>& sm, TileRegs<KD, KV>& R) {
  using WG = WinGeom<KD>;
  constexpr int D = KD * 32;
  const int r = threadIdx.x / WG::TPR, c0 = threadIdx.x % WG::TPR;
  const int row = key0 + r < key_end ? sm.sidx[key0 - key_begin + r] : -1;
  R.row = row;
  const uint16_t* src = row >= kNewRow ? a.x_new + (int64_t)(row - kNewRow) * D : a.win + (int64_t)max(row, 0) * D;
  const int nu = rope0 >> 3;  // unrotated chunks
#pragma unroll
  for (int i = 0; i < WG::NC; ++i) R.v[i] = *reinterpret_cast<const uint4*>(src + 8 * min(c0 + WG::TPR * i, WG::CPR - 1));
  R.rot = *reinterpret_cast<const uint4*>(src + min(rope0 + 8 * c0, D - 8));
  (void)nu;
}

// Window rows into the bf16 tile; the rotated chunk is rotated at the token's position here, the
// remainder going to klo.
template <int KD, int KV>
__device__ __forceinline__ void window_store(const AttnArgs& a, const KeySpace& ks, int key0, int rope0,
                                             AttnSmem<KD>& sm, const TileRegs<KD, KV>& R) {
  using WG = WinGeom<KD>;
  constexpr int D = KD * 32;
  const int r = threadIdx.x / WG::TPR, c0 = threadIdx.x % WG::TPR;
  const int nu = rope0 >> 3;
  const bool ok = R.row >= 0;
#pragma unroll
  for (int i = 0; i < WG::NC; ++i) {
    const int ch = c0 + WG::TPR * i;
    if (ch < nu) *reinterpret_cast<uint4*>(&sm.t.b.k16[r][8 * ch]) = ok ? R.v[i] : make_uint4(0, 0, 0, 0);
  }
  if (8 * c0 < a.d_rope) {
    uint4 hi = make_uint4(0, 0, 0, 0), lo = hi;
    if (ok) rope8_hi_lo(R.rot, ks.w0 + (key0 + r - ks.n_c), a.rev_freq, 4 * c0, &hi, &lo);
    const int d0 = rope0 + 8 * c0;
    *reinterpret_cast<uint4*>(&sm.t.b.k16[r][d0]) = hi;
    *reinterpret_cast<uint4*>(&sm.t.b.klo[r][d0 - (D - 64)]) = lo;
  }
  if (c0 == 0) {
    sm.kscale[r] = ok ? a.scale_log2 : -INFINITY;
    sm.kvscale[r] = ok ? 1.f : 0.f;
  }
}

// Per-wave online-softmax state for heads 4g..4g+3 of the lane's group. m is the exponent base
// of the running sums; it may lag the true running maximum by up to kRescaleSlack (p <= 2^8),
// so O is rescaled only when a logit exceeds it by more than that. l holds this wave's keys only.
template <int NO>
struct WaveState {
  f32x4 o[NO];
  float m[4], l[4];
};

// S for keys [16w, 16w + 16) of the tile staged in LDS. F8: fp8 rows; WIN: window rows (key
// remainders of the last 64 dims in klo). The rotated dims (d_rope <= 64) lie in the last two
// 32-dim blocks, whose query remainders (qlo) and window-key remainders are zero outside them.
template <int KD, bool F8, bool WIN>
__device__ __forceinline__ f32x4 tile_qk(const AttnSmem<KD>& sm, const uint4* qa, const uint4* qlo) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int krow = 16 * w + col;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int BQ = 3;  // operand reads in flight ahead of the MFMAs
  constexpr int RB0 = KD >= kRB ? KD - kRB : 0;  // first block that may hold rotated dims
#pragma unroll
  for (int s0 = 0; s0 < KD; s0 += BQ) {
    bf16x8 kb[BQ];
#pragma unroll
    for (int u = 0; u < BQ; ++u) {
      const int s = s0 + u;
      if (s < KD) {
        if constexpr (F8) {
          const uint2 v = *reinterpret_cast<const uint2*>(&sm.t.k8[krow][32 * s + 8 * g]);
          kb[u] = fp8x8_to_bf16(v.x, v.y);
        } else {
          kb[u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sm.t.b.k16[krow][32 * s + 8 * g]));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < BQ; ++u) {
      const int s = s0 + u;
      if (s < KD) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[s]), kb[u], acc, 0, 0, 0);
        if (s >= RB0) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qlo[s - RB0]), kb[u], acc, 0, 0, 0);
          if constexpr (WIN) {
            const bf16x8 kl = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4*>(&sm.t.b.klo[krow][32 * (s - RB0) + 8 * g]));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[s]), kl, acc, 0, 0, 0);
          }
        }
      }
    }
  }
  return acc;
}

// O += P V over the staged tile (NKS steps of 32 keys) for this wave's value dims. P (A operand):
// lane (head col, group g) holds keys 8g..8g+7 of a step; V (B operand): lane (dim col, group g)
// holds the same keys of its dim.
template <int KD, int NO, bool F8, int NKS, int NVB>
__device__ __forceinline__ void tile_pv(const AttnSmem<KD>& sm, WaveState<NO>& st) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  constexpr bool kEven = NO * 4 == NVB;  // every wave owns NO value dim blocks
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int kb0 = 32 * ks + 8 * g;
    bf16x8 pa;
    {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&sm.pt[kb0 + (col >> 2)][4 * (col & 3)]));
      const i16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&sm.pt[kb0 + 4 + (col >> 2)][4 * (col & 3)]));
      pa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    constexpr int BV = 4;
#pragma unroll
    for (int n0 = 0; n0 < NO; n0 += BV) {
      bf16x8 vb[BV];
#pragma unroll
      for (int u = 0; u < BV; ++u) {
        const int n = n0 + u;
        const int nb = w * NO + n;  // value dim block of this wave
        if (n < NO && (kEven || nb < NVB)) {
          if constexpr (F8) {
            const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2*)(&sm.t.k8[kb0 + (col >> 1)][16 * nb + 8 * (col & 1)]));
            vb[u] = fp8x8_to_bf16((uint32_t)v.x, (uint32_t)v.y);
          } else {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(&sm.t.b.k16[kb0 + (col >> 2)][16 * nb + 4 * (col & 3)]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(&sm.t.b.k16[kb0 + 4 + (col >> 2)][16 * nb + 4 * (col & 3)]));
            vb[u] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
      }
#pragma unroll
      for (int u = 0; u < BV; ++u) {
        const int n = n0 + u;
        if (n < NO && (kEven || w * NO + n < NVB))
          st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb[u], st.o[n], 0, 0, 0);
      }
    }
  }
}

// Softmax of one staged tile of TK keys (wave w owns keys [16w, 16w+16) when 16w < TK): tile maxima
// through LDS, the exponent base moved when needed (every wave rescales its O), P^T to LDS.
// Ends with the barrier that makes P^T visible.
template <int KD, int NO>
__device__ __forceinline__ void tile_softmax(AttnSmem<KD>& sm, WaveState<NO>& st, const f32x4& s, int TK) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int krow = 16 * w + col;
  const bool active = 16 * w < TK;
  float x[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (active) {
    const float ck = sm.kscale[krow];
    const f32x4 qs = *reinterpret_cast<const f32x4*>(&sm.qscale[4 * g]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = ck == -INFINITY ? -INFINITY : s[r] * qs[r] * ck;
      const float m_ = row16_max(x[r]);
      if (col == 0) sm.xmax[w][4 * g + r] = m_;
    }
  }
  __syncthreads();
  const int nk = TK / 16;
  bool need = false;
  float mx[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mx[r] = sm.xmax[0][4 * g + r];
    for (int j = 1; j < nk; ++j) mx[r] = fmaxf(mx[r], sm.xmax[j][4 * g + r]);
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
    for (int n = 0; n < NO; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st.o[n][r] *= alpha[r];
    }
  }
  if (active) {
    const float vk = sm.kvscale[krow];
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float base = st.m[r] == -INFINITY ? 0.f : st.m[r];
      const float p = exp2f(x[r] - base);
      st.l[r] += row16_sum(p);
      pv[r] = p * vk;  // value-side scale folded into P
    }
    uint2 wv;
    wv.x = pack_bf16x2(pv[0], pv[1]);
    wv.y = pack_bf16x2(pv[2], pv[3]);
    *reinterpret_cast<uint2*>(&sm.pt[krow][4 * g]) = wv;
  }
  __syncthreads();
}

template <int KD, int NVB, int KV>
__global__ __launch_bounds__(kNT, 2) void attn_kernel(AttnArgs a) {
  constexpr int D = KD * 32;
  constexpr int NO = (NVB + 3) / 4;  // value dim blocks per wave
  constexpr bool F8 = KV == kKvFp8;
  constexpr int TKE = F8 ? kTK8 : kTK16;
  __shared__ AttnSmem<KD> sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
  const int g = lane >> 4, col = lane & 15;

  // work item (query, head group, split); with xcd_map the items of a query are contiguous in
  // the order of one XCD's workgroups (workgroups go round-robin to the 8 XCDs)
  const int total = a.nq * a.n_hg * a.n_splits;
  const int item = a.xcd_map ? (int)(blockIdx.x & 7) * (total >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int split = item % a.n_splits;
  const int qh = item / a.n_splits;
  const int hg = qh % a.n_hg, qi = qh / a.n_hg;
  const int h0 = hg * kHG;
  const int rope0 = D - a.d_rope;
  constexpr int RB0 = KD >= kRB ? KD - kRB : 0;  // first block that may hold rotated dims

  // the query's raw dims: requested first, they depend on nothing else
  uint4 qa[KD], qlo[kRB];
  const int h = h0 + col;
#pragma unroll
  for (int s = 0; s < KD; ++s) {
    const int d0 = 32 * s + 8 * g;
    qa[s] = h < a.H ? *reinterpret_cast<const uint4*>(a.q + ((int64_t)qi * a.H + h) * D + d0) : make_uint4(0, 0, 0, 0);
  }
  qlo[0] = qlo[1] = make_uint4(0, 0, 0, 0);

  const KeySpace ks = key_space(a, qi);
  const int n_keys = ks.n_c + ks.n_w;
  const int key_begin = split * a.keys_per_split;
  const int key_end = min(n_keys, key_begin + a.keys_per_split);
  const int e_end = min(key_end, ks.n_c);  // entry keys [key_begin, e_end), window keys after
  const int w_begin = max(key_begin, ks.n_c);
  // the rows of this split's keys: entry rows in the sequence's cache (top-k slot or dense
  // index; out of range = masked), then window rows in win (ring slot or prompt row)
  {
    const int64_t wseq = a.ring ? (int64_t)(qi / a.q_per_seq) * a.ring_cap : -a.pos0;
    const int64_t wbase = a.ring ? ks.w0 % a.ring_cap : ks.w0;  // row of window key 0 before wrapping
    // append mode: positions from the sequence's first query on are the step's new tokens
    const int j = qi % a.q_per_seq;
    const int64_t t_new = a.x_new ? ks.t - j : INT64_MAX;
    for (int i = tid; i < key_end - key_begin; i += kNT) {
      const int key = key_begin + i;
      int row;
      if (key < ks.n_c) {
        row = a.topk ? a.topk[(int64_t)qi * a.k + key] : key;
        if (row >= a.N_cap) row = -1;
      } else if (ks.w0 + (key - ks.n_c) >= t_new) {
        row = kNewRow + (qi - j) + (int)(ks.w0 + (key - ks.n_c) - t_new);
      } else {
        int64_t slot = wbase + (key - ks.n_c);
        if (a.ring && slot >= a.ring_cap) slot -= a.ring_cap;  // n_w <= W <= ring_cap
        row = (int)(wseq + slot);
      }
      sm.sidx[i] = row;
    }
    // one workgroup per sequence writes the new tokens to the ring
    if (a.x_new && j == 0 && split == 0 && hg == 0)
      append_new_tokens(a.x_new, a.z_new, a.ring_w, a.ring_z, qi, a.q_per_seq, ks.t, a.ring_cap, a.D, tid, kNT);
  }
  if (tid < kTK16) {  // window remainders of the last 64 dims below rope0 are zero
    for (int d = D - 64; d < rope0; ++d)
      if (d >= 0) sm.t.b.klo[tid][d - (D - 64)] = 0;
  }
  __syncthreads();  // sidx ready

  const int64_t seq = (int64_t)(a.ckv_seq ? qi / a.q_per_seq : 0) * a.ckv_seq;
  constexpr int row_bytes = KV == kKvBf16 ? 2 * D : (KV == kKvFp8 ? D : D / 2);
  constexpr int srow_bytes = KV == kKvFp8 ? 4 : (KV == kKvMxfp4 ? D / 32 : 0);
  const uint8_t* cbase = reinterpret_cast<const uint8_t*>(a.ckv) + seq * row_bytes;
  const uint8_t* sbase = a.ckv_scale ? reinterpret_cast<const uint8_t*>(a.ckv_scale) + seq * srow_bytes : nullptr;

  // the split's first tile is requested before the query rotation, whose arithmetic then
  // overlaps the loads
  const bool has_e = key_begin < e_end;
  TileRegs<KD, KV> RT;
  if (has_e)
    entry_load<KD, KV>(cbase, sbase, key_begin, e_end, key_begin, sm, RT);
  else if (w_begin < key_end)
    window_load<KD, KV>(a, w_begin, key_end, key_begin, rope0, sm, RT);

  // the query's rotated dims: each of the 16 heads x d_rope/8 chunks rotated once at t (a bf16
  // value and a bf16 remainder) into LDS
  {
    const int rc = a.d_rope >> 3;
    if ((int)tid < kHG * rc) {
      const int hl = tid / rc, ch = tid - hl * rc;
      const int hh = h0 + hl;
      uint4 hi = make_uint4(0, 0, 0, 0), lo = hi;
      if (hh < a.H) {
        const uint4 v = *reinterpret_cast<const uint4*>(a.q + ((int64_t)qi * a.H + hh) * D + rope0 + 8 * ch);
        rope8_hi_lo(v, ks.t, a.rev_freq, 4 * ch, &hi, &lo);
      }
      *reinterpret_cast<uint4*>(&sm.qrh[hl][8 * ch]) = hi;
      *reinterpret_cast<uint4*>(&sm.qrl[hl][8 * ch]) = lo;
    }
  }
  float ss = 0.f;  // sum of squares of the raw query over this lane's dims (RMSNorm)
  if (a.q_rms_eps > 0.f) {
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      float f[8];
      unpack8(qa[s], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    }
  }
  // query RMSNorm factor per head (applied to the logits): 1 / sqrt(mean(q^2) + eps)
  {
    ss += __shfl_xor(ss, 16, kWave);
    ss += __shfl_xor(ss, 32, kWave);
    const float r = a.q_rms_eps > 0.f ? 1.0f / sqrtf(ss / (float)D + a.q_rms_eps) : 1.0f;
    if (w == 0 && g == 0) sm.qscale[col] = r;
  }
  __syncthreads();  // rotated query dims ready
#pragma unroll
  for (int s = 0; s < KD; ++s) {
    const int d0 = 32 * s + 8 * g;
    if (d0 >= rope0) {
      qa[s] = *reinterpret_cast<const uint4*>(&sm.qrh[col][d0 - rope0]);
      const uint4 lo = *reinterpret_cast<const uint4*>(&sm.qrl[col][d0 - rope0]);
      if (s == RB0)
        qlo[0] = lo;
      else
        qlo[1] = lo;
    }
  }

  WaveState<NO> st;
#pragma unroll
  for (int n = 0; n < NO; ++n) st.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    st.m[r] = -INFINITY;
    st.l[r] = 0.f;
  }

  // phase 1: compressed entries
  if (has_e) {
    for (int key0 = key_begin; key0 < e_end; key0 += TKE) {
      __syncthreads();  // the previous tile's reads are done
      entry_store<KD, KV>(a, sm, RT);
      __syncthreads();
      if (key0 + TKE < e_end)
        entry_load<KD, KV>(cbase, sbase, key0 + TKE, e_end, key_begin, sm, RT);
      else if (w_begin < key_end)
        window_load<KD, KV>(a, w_begin, key_end, key_begin, rope0, sm, RT);
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      if (16 * w < TKE) s = tile_qk<KD, F8, false>(sm, qa, qlo);
      tile_softmax<KD, NO>(sm, st, s, TKE);
      tile_pv<KD, NO, F8, TKE / 32, NVB>(sm, st);
    }
  }
  // phase 2: window tokens
  for (int key0 = w_begin; key0 < key_end; key0 += kTK16) {
    __syncthreads();
    window_store<KD, KV>(a, ks, key0, rope0, sm, RT);
    __syncthreads();
    if (key0 + kTK16 < key_end) window_load<KD, KV>(a, key0 + kTK16, key_end, key_begin, rope0, sm, RT);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if (16 * w < kTK16) s = tile_qk<KD, false, true>(sm, qa, qlo);
    tile_softmax<KD, NO>(sm, st, s, kTK16);
    tile_pv<KD, NO, false, 1, NVB>(sm, st);
  }

  // the key sums of the waves (same exponent base): l = sum over waves
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.lsum[w][4 * g + r] = st.l[r];
  }
  __syncthreads();
  float lt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    lt[r] = sm.lsum[0][4 * g + r] + sm.lsum[1][4 * g + r] + sm.lsum[2][4 * g + r] + sm.lsum[3][4 * g + r];

  if (a.n_splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hr = h0 + 4 * g + r;
      if (hr >= a.H) continue;
      const float inv = lt[r] > 0.f ? 1.f / lt[r] : 0.f;
      uint16_t* dst = a.out + ((int64_t)qi * a.H + hr) * a.d_v;
#pragma unroll
      for (int n = 0; n < NO; ++n) {
        const int nb = w * NO + n;
        if (nb < NVB) dst[16 * nb + col] = (uint16_t)f32_to_bf16_rne(st.o[n][r] * inv);
      }
      if (a.out_lse && col == 0 && w == 0)
        a.out_lse[(int64_t)qi * a.H + hr] = lt[r] > 0.f ? (st.m[r] + log2f(lt[r])) * kLn2 : -INFINITY;
    }
    return;
  }

  // split partial: unnormalised O, exponent base and sum
  const int64_t pbase = ((int64_t)qh * a.n_splits + split) * kHG;  // first head row of this split
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float* dst = a.part_o + (pbase + 4 * g + r) * a.d_v;
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      const int nb = w * NO + n;
      if (nb < NVB) dst[16 * nb + col] = st.o[n][r];
    }
    if (col == 0 && w == 0) {
      a.part_ml[(pbase + 4 * g + r) * 2 + 0] = st.m[r];
      a.part_ml[(pbase + 4 * g + r) * 2 + 1] = lt[r];
    }
  }
}

// One workgroup per (query, head): log-sum-exp merge of the split partials. Thread t owns dims
// 4t..4t+3 (d_v <= 4 * kMergeNT). Split rows are read kMergeBatch at a time, the batch requested
// before the previous one is summed; rows past the last split repeat it with weight 0, so every
// load is unconditional.
constexpr int kMergeNT = 128;
constexpr int kMergeBatch = 8;
__global__ __launch_bounds__(kMergeNT) void attn_merge_kernel(AttnArgs a) {
  __shared__ float wsh[kMaxSplits + kMergeBatch];
  __shared__ float red[2];
  const int qi = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int S = a.n_splits;
  const int64_t row0 = ((int64_t)(qi * a.n_hg + h / kHG) * S) * kHG + h % kHG;  // split s: row0 + s * kHG
  const int dd = min(4 * tid, a.d_v - 4);  // threads past d_v read the last dims and store nothing
  if (tid < kWave) {
    float mx = -INFINITY;
    for (int sp = tid; sp < S; sp += kWave) mx = fmaxf(mx, a.part_ml[(row0 + (int64_t)sp * kHG) * 2]);
    mx = wave_max(mx);
    const float Mb = mx == -INFINITY ? 0.f : mx;
    float l = 0.f;
    for (int sp = tid; sp < S + kMergeBatch; sp += kWave) {
      float wt = 0.f;
      if (sp < S) {
        const float2 ml = *reinterpret_cast<const float2*>(&a.part_ml[(row0 + (int64_t)sp * kHG) * 2]);
        wt = exp2f(ml.x - Mb);
        l += wt * ml.y;
      }
      wsh[sp] = wt;
    }
    l = wave_sum(l);
    if (tid == 0) {
      red[0] = Mb;
      red[1] = l;
    }
  }
  __syncthreads();
  const float Mb = red[0], L = red[1];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto fetch = [&](f32x4 (&v)[kMergeBatch], int s0) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      v[u] = *reinterpret_cast<const f32x4*>(a.part_o + (row0 + (int64_t)min(s0 + u, S - 1) * kHG) * a.d_v + dd);
  };
  auto sum = [&](const f32x4 (&v)[kMergeBatch], int s0) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) acc += wsh[s0 + u] * v[u];
  };
  f32x4 v0[kMergeBatch], v1[kMergeBatch];
  fetch(v0, 0);
  for (int s0 = 0;; s0 += 2 * kMergeBatch) {  // v0 holds rows s0.. on entry
    if (s0 + kMergeBatch >= S) {
      sum(v0, s0);
      break;
    }
    fetch(v1, s0 + kMergeBatch);
    sum(v0, s0);
    if (s0 + 2 * kMergeBatch >= S) {
      sum(v1, s0 + kMergeBatch);
      break;
    }
    fetch(v0, s0 + 2 * kMergeBatch);
    sum(v1, s0 + kMergeBatch);
  }
  if (4 * tid < a.d_v) {
    uint2 packed;
    packed.x = pack_bf16x2(acc.x * inv, acc.y * inv);
    packed.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(a.out + ((int64_t)qi * a.H + h) * a.d_v + dd) = packed;
  }
  if (tid == 0 && a.out_lse) a.out_lse[(int64_t)qi * a.H + h] = L > 0.f ? (Mb + log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- host side
struct AttnPlan {
  int n_hg, n_splits, keys_per_split;
  size_t ws;  // bytes of the split partials
};

// Splits of a query's key set: about two workgroups per CU over the whole job, each split a
// multiple of 64 keys (whole tiles of either kind), at most kMaxSplitKeys keys and kMaxSplits
// splits.
static AttnPlan plan_attn(int nq, int H, int d_v, int max_keys) {
  AttnPlan p;
  p.n_hg = (H + kHG - 1) / kHG;
  const int64_t base = (int64_t)nq * p.n_hg;
  int splits = (int)(kTargetWG / base);
  if (splits < 1) splits = 1;
  int per = (max_keys + splits - 1) / splits;
  per = (per + 63) / 64 * 64;
  if (per < 64) per = 64;
  const int min_per = (max_keys + kMaxSplits - 1) / kMaxSplits;
  if (per < min_per) per = (min_per + 63) / 64 * 64;
  if (per > kMaxSplitKeys) per = kMaxSplitKeys;
  splits = (max_keys + per - 1) / per;
  if (splits < 1) splits = 1;
  p.n_splits = splits;
  p.keys_per_split = per;
  p.ws = splits > 1 ? (size_t)base * splits * kHG * ((size_t)d_v + 2) * sizeof(float) : 0;
  return p;
}

typedef void (*AttnKernel)(AttnArgs);

template <int KV>
static AttnKernel pick_dims(int D, int d_v) {
  if (D == 576 && d_v == 512) return attn_kernel<18, 32, KV>;
  if (D == 128 && d_v == 128) return attn_kernel<4, 8, KV>;
  if (D == 64 && d_v == 32) return attn_kernel<2, 2, KV>;
  if (D == 256 && d_v == 128) return attn_kernel<8, 8, KV>;
  return nullptr;
}

// Compiled (D, d_v) pairs.
static AttnKernel pick_kernel(int D, int d_v, int kv) {
  return kv == kKvFp8 ? pick_dims<kKvFp8>(D, d_v)
                      : (kv == kKvMxfp4 ? pick_dims<kKvMxfp4>(D, d_v) : pick_dims<kKvBf16>(D, d_v));
}

static int launch_attn(const char* name, AttnArgs a, const AttnPlan& p, void* ws, size_t ws_bytes, hipStream_t s) {
  for (int i = 0; i < a.d_rope / 2; ++i)
    a.rev_freq[i] = pow((double)a.rope_base, -2.0 * (double)i / (double)a.d_rope) / 6.283185307179586476925286766559;
  CSKV_REQUIRE(p.ws == 0 || (ws && ws_bytes >= p.ws), CSKV_EWORKSPACE, "%s: workspace %zu < %zu bytes", name,
               ws_bytes, p.ws);
  a.n_hg = p.n_hg;
  a.n_splits = p.n_splits;
  a.keys_per_split = p.keys_per_split;
  CSKV_REQUIRE(p.n_splits <= kMaxSplits, CSKV_ENOTSUP, "%s: %d key splits > %d (key set too large)", name,
               p.n_splits, kMaxSplits);
  CSKV_REQUIRE(p.n_splits == 1 || a.d_v <= 4 * kMergeNT, CSKV_ENOTSUP, "%s: d_v=%d > %d with split keys", name,
               a.d_v, 4 * kMergeNT);
  if (p.n_splits > 1) {
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = a.part_o + (size_t)a.nq * p.n_hg * p.n_splits * kHG * a.d_v;
  }
  const int64_t total = (int64_t)a.nq * p.n_hg * p.n_splits;
  CSKV_REQUIRE(total < (1ll << 31), CSKV_ENOTSUP, "%s: %lld workgroups", name, (long long)total);
  a.xcd_map = total % 8 == 0 ? 1 : 0;
  AttnKernel kern = pick_kernel(a.D, a.d_v, a.kv_dtype);
  hipLaunchKernelGGL(kern, dim3((unsigned)total), dim3(kNT), 0, s, a);
  CSKV_LAUNCH_CHECK(name);
  if (p.n_splits > 1) {
    hipLaunchKernelGGL(attn_merge_kernel, dim3(a.nq, a.H), dim3(kMergeNT), 0, s, a);
    CSKV_LAUNCH_CHECK(name);
  }
  return CSKV_OK;
}

// ---------------------------------------------------------------- entry from attention.hip
size_t ws_bytes(int nq, int H, int d_v, int max_keys) { return plan_attn(nq, H, d_v, max(max_keys, 1)).ws; }

int launch(const char* name, const AttnCall& c, void* ws, size_t ws_bytes, hipStream_t s) {
  AttnArgs a{};
  a.q = c.q;
  a.q_pos = c.q_pos;
  a.pos0 = c.pos0;
  a.ckv = c.ckv;
  a.ckv_scale = c.ckv_scale;
  a.kv_dtype = c.kv_dtype;
  a.N_cap = c.N_cap;
  a.ckv_seq = c.ckv_seq;
  a.n_entries = c.n_entries;
  a.m = c.m;
  a.topk = c.topk;
  a.k = c.k;
  a.win = c.win;
  a.x_new = c.x_new;
  a.z_new = c.z_new;
  a.ring_w = const_cast<uint16_t*>(c.win);  // written only in append mode, whose caller passes a writable ring
  a.ring_z = c.ring_z;
  a.ring = c.ring;
  a.ring_cap = c.ring_cap;
  a.q_per_seq = c.q_per_seq;
  a.W = c.W;
  a.nq = c.nq;
  a.H = c.H;
  a.D = c.D;
  a.d_rope = c.d_rope;
  a.d_v = c.d_v;
  a.rope_base = c.rope_base;
  a.scale_log2 = c.scale_log2;
  a.q_rms_eps = c.q_rms_eps;
  a.out = c.out;
  a.out_lse = c.out_lse;
  const int max_keys = (c.N_cap > 0 ? (c.topk ? c.k : c.N_cap) : 0) + c.W;
  return launch_attn(name, a, plan_attn(c.nq, c.H, c.d_v, max(max_keys, 1)), ws, ws_bytes, s);
}

}  // namespace g16
}  // namespace cskv
