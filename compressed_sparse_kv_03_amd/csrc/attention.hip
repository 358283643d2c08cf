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
// Design. A workgroup of eight waves takes one query, a block of 64 heads and one
// contiguous split of the query's key set (compressed entries, then window
// tokens); one workgroup runs per CU. Keys go through LDS 64 at a time: fp8
// entries as their raw codes in a three-tile ring filled by direct global-to-LDS
// loads two tiles ahead, bf16 and MXFP4 entries and window tokens as bf16 rows
// staged through registers (MXFP4 widened exactly, window tokens rotated at their
// own position). Every product is a v_mfma_f32_32x32x16_bf16 with the keys or the
// value dims as rows and 32 heads as columns, so each K and V element read from
// LDS serves 32 heads and each lane owns one head:
//   S^T = K Q^T: wave (hh, kh, dq) takes heads [32hh, 32hh+32), keys
//     [32kh, 32kh+32) and one half of the dims (the halves balance the MFMA
//     count); the query's dims stay in registers for the whole split (B operand);
//   softmax in the log2 domain per head: the two dim halves of a block hand each
//     other half of their partial logits through LDS, the key halves meet in LDS;
//     P^T goes to LDS as [head][key];
//   O^T += V^T P^T: wave (hh, vq) takes heads [32hh, 32hh+32) and a quarter of
//     the value dims; V^T is read with the transposed LDS reads ds_read_b64_tr_b8
//     (fp8 codes, widened in registers) or ds_read_b64_tr_b16 (bf16 rows).
// The rotated dims of the query and of window keys carry 16 significant bits:
// they are split into a bf16 value and a bf16 remainder and both go through the
// MFMA (for entry keys, stored exactly, the query remainder only), so the
// rotation adds no bf16 rounding to the logits.
// A query's splits write their normalised partial outputs O / l in fp16 with
// (max, sum) in fp32, and a second launch merges them (log-sum-exp merge; merging
// in the last split to finish needs a device-scope release per workgroup, an L2
// write-back that costs about what the launch does). One split writes the output
// directly. Short key sets of few queries go to the 16-head kernel instead
// (attention_g16.hip).
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attention_call.h"
#include "common.cuh"
#include "host_util.h"

namespace cskv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kNT = 512;             // threads per workgroup (8 waves)
constexpr int kHB = 64;              // heads per workgroup
constexpr int kTK = 64;              // keys per tile
constexpr int kTPR = kNT / kTK;      // staging threads per key row
constexpr int kMaxRopePairs = 32;
constexpr int kMaxSplitKeys = 2048;  // key rows listed per split
constexpr int kMaxSplits = 64;
constexpr int kCUs = 256;            // one workgroup per CU (the default CU budget of a split plan)
constexpr int kMergeTiles = 2;       // the merge launch, in tile times (split planning)
constexpr int kWgFixedTiles = 2;     // a workgroup's prologue and epilogue, in tile times
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;  // log2 units the running max may run ahead of the exponent base


struct AttnArgs {
  // the fields a workgroup reads before its first loads, packed at the front of the argument block
  const uint16_t* q;         // [nq, H, D]
  const int64_t* q_pos;      // [nq] (decode) or nullptr (prefill: pos0 + row)
  const int32_t* n_entries;  // [nq] (decode) or nullptr (prefill: min(N, (t+1)/m))
  const int32_t* topk;       // [nq, k] or nullptr (dense)
  const void* ckv;           // [B_kv, N_cap, D] bf16 bits, fp8 codes, or MXFP4 codes [.., D/2]
  const void* ckv_scale;     // fp32 [B_kv, N_cap] (fp8) or E8M0 bytes [B_kv, N_cap, D/32] (MXFP4)
  int64_t ckv_seq;           // entries between sequences (0: all queries share one cache)
  int64_t pos0;
  double rope_step;          // base^(-2 / d_rope): ratio of consecutive RoPE frequencies (host fp64)
  int N_cap;
  int q_per_seq;             // consecutive queries sharing one sequence's ring and cache (decode)
  int H;
  int n_hb;                  // head blocks of 64
  int n_splits, keys_per_split;
  int n_esplits;             // n_esplits < n_splits: splits [0, n_esplits) take keys_per_split entry keys
                             // each, the rest win_per_split window keys each; else all keys in order
  int win_per_split;
  int k, m, W;
  int ring;                  // 1 (decode, q_pos and n_entries given): slot = pos mod ring_cap of sequence
                             // qi / q_per_seq; 0 (prefill): row = pos - pos0 of x
  float q_rms_eps;           // > 0: unit-gain RMSNorm of each query head (folded into its logits)
  // the rest
  const uint16_t* win;       // decode: rings [B, R, D]; prefill: x [T, D]
  int kv_dtype;              // kKvBf16, kKvFp8 or kKvMxfp4
  int ring_cap;
  int nq, D, d_rope, d_v;
  float scale_log2;          // softmax_scale * log2(e)
  uint16_t* out;             // [nq, H, d_v]
  float* out_lse;            // [nq, H]
  uint16_t* part_o;          // [nq, n_hb, n_splits, 64, d_v] fp16: the split's O / l
  float* part_ml;            // [nq, n_hb, n_splits, 64, 2]: exponent base m, sum l
  const uint16_t* x_new;     // append mode: [B, T, D] new tokens (rows >= kNewRow), else nullptr
  const float* z_new;        // [B, T] or nullptr
  uint16_t* ring_w;          // the rings (win), written in append mode
  float* ring_z;             // [B, R] (with z_new)
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
  // decode: the query's position and its entry count are requested together, before either is
  // used (one memory round trip instead of two)
  const bool by_count = a.ring && a.N_cap != 0 && a.topk == nullptr;
  int64_t t = a.pos0 + qi;
  int n = 0;
  if (by_count) {
    n = a.n_entries[qi];
    t = a.q_pos[qi];
  } else if (a.ring) {
    t = a.q_pos[qi];
  }
  ks.t = t;
  if (a.N_cap == 0) {
    ks.n_c = 0;  // no cache (every top-k slot would be masked)
  } else if (a.topk) {
    ks.n_c = a.k;
  } else if (by_count) {
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

// cos / sin of the RoPE angle pos * inv_freq, with rev = inv_freq / (2 pi) (fp64): the angle
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
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  uint4 v;
  v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return v;
}

// Two floats to packed bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Two floats to packed fp16 with round-to-nearest-even.
__device__ __forceinline__ uint32_t cvt_f16x2(float lo, float hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// v if ok, else zeros (component selects on values, so that register arrays stay in registers)
__device__ __forceinline__ uint4 keep_if(bool ok, const uint4 v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// LDS. fp8 entry tiles live in a ring of kStages tiles of codes, chunk-major ([16-byte chunk of
// dims][key][16 bytes]: a wave-wide request fills one chunk of all 64 keys, and the MFMA operand
// reads and transposed reads touch consecutive 16-byte slots), filled by direct global-to-LDS
// loads two tiles ahead of use; the per-entry scales beside them. bf16 tiles
// (window tokens; bf16 and MXFP4 entries) overlay the ring: rows of D + 8 elements, and klo, window
// keys' remainders of the last 64 dims (zero where not rotated). Rows are 16 bytes apart modulo
// 256, so the MFMA operand reads and the transposed reads are free of bank conflicts. P^T is
// [head][key]; xs carries the half of a block's partial logits that the other wave of the block
// needs.
constexpr int kStages = 3;
template <int D>
struct AttnSmem {
  union {
    struct {
      __align__(16) uint8_t k8[kStages][D / 16][kTK][16];
      __align__(16) float sc[kStages][kTK];
    } r;
    struct {
      __align__(16) uint16_t k[kTK][D + 8];
      __align__(16) uint16_t klo[kTK][64 + 8];
      __align__(16) uint8_t k4[D / 32][kTK][16];  // MXFP4 entries: e2m1 codes, 32-dim block major
      uint8_t s4[kTK][D / 32];                    // and their E8M0 block exponents
    } b;
  } t;
  __align__(16) uint16_t p[kHB][kTK + 8];
  __align__(16) f32x4 xs[8][2][kWave];
  float xmax[4][kHB];
  float lsum[4][kHB];
  float qss[2][kHB];                 // query sums of squares over each half of the dims
  int rescale;                       // a tile's logit exceeded its head's exponent base by more than the slack
  double rev[kMaxRopePairs];         // RoPE frequencies (revolutions per position)
  int sidx[kMaxSplitKeys];
};

// ---------------------------------------------------------------- fp8 entry tiles: direct loads
// A wave-wide request of 16 (4) bytes per lane from gp into LDS at lds + 16 * lane (4 * lane),
// the LDS address taken from M0. Nothing is written to registers; the data lands asynchronously
// and is waited for with s_waitcnt vmcnt, whose count these requests advance in issue order.
// m0 is named as clobbered; the compiler warns that, being reserved, it may not be preserved
// around the statement. No compiler-generated code in these kernels uses m0 (it appears in the
// generated assembly only in these statements), so nothing of the compiler's is live in it.
__device__ __forceinline__ void dma16(const void* gp, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gp) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gp, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(gp) : "memory", "m0");
}
// x combined with the x of the lane 32 apart, on the VALU: a permlane32 swap of two copies of x
// leaves x[l] in one result and x[l ^ 32] in the other, in every lane (no LDS round trip as for
// a shuffle).
__device__ __forceinline__ float add_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
// The wave's index in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// s_waitcnt with only the vector-memory count: vmcnt <= n (n < 16)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

// One fp8 tile is D/16 wave-wide chunk requests (lane = key) plus one request for the scales,
// request i issued by wave i % 8.
template <int D>
struct RingGeom {
  static constexpr int NCH = D / 16;          // chunk requests
  static constexpr int NREQ = NCH + 1;        // then the scale request
  static constexpr int reqs(int w) { return w < NREQ ? (NREQ - 1 - w) / 8 + 1 : 0; }
};

// Requests tile rows [key0, key0 + 64) of the split (entry rows from sidx; a masked key or a key
// past e_end reads row 0, which the validity mask hides) into ring stage `stage`. Every lane of
// every wave takes part in each of its wave's requests, so the count per wave is fixed.
template <int D>
__device__ __forceinline__ void issue_tile_f8(AttnSmem<D>& sm, int stage, const uint8_t* cbase, const float* sbase,
                                              int key0, int e_end, int key_begin, bool dense) {
  using G = RingGeom<D>;
  const int lane = threadIdx.x & (kWave - 1), w = wave_id();
  const uint32_t base = lds_addr(&sm.t.r.k8[stage][0][0][0]);
  const int key = key0 + lane;
  const int row = max(key < e_end ? (dense ? key : sm.sidx[key - key_begin]) : -1, 0);  // dense: entry = key
  const uint8_t* src = cbase + (int64_t)row * D;
#pragma unroll
  for (int j = 0; j < (G::NREQ + 7) / 8; ++j) {
    const int i = w + 8 * j;
    if (i < G::NCH)
      dma16(src + 16 * i, __builtin_amdgcn_readfirstlane(base + 1024u * (uint32_t)i));
    else if (i == G::NCH)
      dma4(sbase + row, __builtin_amdgcn_readfirstlane(lds_addr(&sm.t.r.sc[stage][0])));
  }
}

// Waits for this wave's requests of the current tile: `later` says whether the next tile's
// requests were issued after them (they may stay in flight).
template <int D>
__device__ __forceinline__ void wait_tile_f8(bool later) {
  using G = RingGeom<D>;
  const int w = wave_id();
  if (!later) {
    wait_vm<0>();
    return;
  }
  switch (G::reqs(w)) {  // the count is wave-uniform; each case is an immediate
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    default: wait_vm<0>(); break;
  }
}

// Validity of the tile's 64 keys (key0 + lane < end and its row listed), the same in every wave.
template <int D>
__device__ __forceinline__ uint64_t tile_mask(const AttnSmem<D>& sm, int key0, int end, int key_begin) {
  const int lane = threadIdx.x & (kWave - 1);
  const int key = key0 + lane;
  const bool ok = key < end && sm.sidx[key - key_begin] >= 0;
  return __ballot(ok);
}

// ---------------------------------------------------------------- bf16 tiles: register staging
// One tile's raw rows in registers. Thread t owns row t / kTPR of the tile and its 16-byte chunks
// t % kTPR + kTPR i (an MX block of 32 dims with its exponent byte for MXFP4), so it looks its row
// up once and issues its loads from one base address. bf16 and MXFP4 entry tiles and window tiles
// (at most two per query) are loaded when they are staged.
template <int D, int KV>
struct EntryGeom {
  static constexpr int CPR = KV == kKvBf16 ? D / 8 : D / 32;  // chunks per row
  static constexpr int NC = (CPR + kTPR - 1) / kTPR;          // chunks per thread
};
template <int D>
struct WinGeom {
  static constexpr int CPR = D / 8;
  static constexpr int NC = CPR / kTPR;  // D % 64 == 0; the last one holds the last 64 dims
};
template <int D, int KV>
struct TileRegs {
  uint4 v[EntryGeom<D, KV>::NC];
  uint32_t bs[KV == kKvMxfp4 ? EntryGeom<D, KV>::NC : 1];
  int row;    // -1: masked
};
template <int D>
struct WinRegs {
  uint4 v[WinGeom<D>::NC];
  int row;
};

// Tile loads. The rows of a split's keys were resolved into sm.sidx (entry row in the cache,
// window row in win, -1 = masked). Loads are unconditional (a masked row reads row 0, a chunk past
// the row end its last chunk); the store writes zeros for a masked row (a masked key gets p = 0,
// which must not meet a non-finite value in the MFMA).
template <int D, int KV>
__device__ __forceinline__ void entry_load(const uint8_t* cbase, const uint8_t* sbase, int key0, int key_end,
                                           int key_begin, const AttnSmem<D>& sm, TileRegs<D, KV>& R) {
  using EG = EntryGeom<D, KV>;
  constexpr int RB = KV == kKvBf16 ? 2 * D : D / 2;  // code bytes per row
  const int r = threadIdx.x / kTPR, c0 = threadIdx.x % kTPR;
  const int row = key0 + r < key_end ? sm.sidx[key0 - key_begin + r] : -1;
  R.row = row;
  const int64_t rr = max(row, 0);
  const uint8_t* src = cbase + rr * RB;
#pragma unroll
  for (int i = 0; i < EG::NC; ++i) {
    const int ch = EG::CPR % kTPR == 0 ? c0 + kTPR * i : min(c0 + kTPR * i, EG::CPR - 1);
    R.v[i] = *reinterpret_cast<const uint4*>(src + 16 * ch);
    if constexpr (KV == kKvMxfp4) R.bs[i] = sbase[rr * (D / 32) + ch];
  }
}

// F4: MXFP4 entries whose keys go through the scaled FP4 MFMA: the codes and block exponents are
// stored as they are (a masked row as code 0, exponent 1.0) and only the value dims (d_v) are
// widened to bf16 rows.
template <int D, int KV, bool F4 = false>
__device__ __forceinline__ void entry_store(AttnSmem<D>& sm, const TileRegs<D, KV>& R, int d_v = D) {
  using EG = EntryGeom<D, KV>;
  const int r = threadIdx.x / kTPR, c0 = threadIdx.x % kTPR;
  const bool ok = R.row >= 0;
#pragma unroll
  for (int i = 0; i < EG::NC; ++i) {
    const int ch = c0 + kTPR * i;
    if (EG::CPR % kTPR != 0 && ch >= EG::CPR) continue;
    if constexpr (F4) {
      *reinterpret_cast<uint4*>(&sm.t.b.k4[ch][r][0]) = keep_if(ok, R.v[i]);
      sm.t.b.s4[r][ch] = ok ? (uint8_t)R.bs[i] : (uint8_t)127;
      if (32 * ch >= d_v) continue;
    }
    if constexpr (KV == kKvBf16) {
      *reinterpret_cast<uint4*>(&sm.t.b.k[r][8 * ch]) = keep_if(ok, R.v[i]);
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
        *reinterpret_cast<uint4*>(&sm.t.b.k[r][32 * ch + 8 * q]) = keep_if(ok, o);
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void window_load(const AttnArgs& a, int key0, int key_end, int key_begin,
                                            const AttnSmem<D>& sm, WinRegs<D>& R) {
  using WG = WinGeom<D>;
  const int r = threadIdx.x / kTPR, c0 = threadIdx.x % kTPR;
  const int row = key0 + r < key_end ? sm.sidx[key0 - key_begin + r] : -1;
  R.row = row;
  const uint16_t* src = row >= kNewRow ? a.x_new + (int64_t)(row - kNewRow) * D : a.win + (int64_t)max(row, 0) * D;
#pragma unroll
  for (int i = 0; i < WG::NC; ++i) R.v[i] = *reinterpret_cast<const uint4*>(src + 8 * (c0 + kTPR * i));
}

// Window rows into the tile: rotated chunks (all in the last 64 dims, held by each thread's last
// chunk) are rotated at the token's position, the bf16 remainder going to klo.
template <int D>
__device__ __forceinline__ void window_store(const AttnArgs& a, const KeySpace& ks, int key0, AttnSmem<D>& sm,
                                             const WinRegs<D>& R) {
  using WG = WinGeom<D>;
  const int r = threadIdx.x / kTPR, c0 = threadIdx.x % kTPR;
  const int rope0 = D - a.d_rope;
  const bool ok = R.row >= 0;
  const uint4 z = make_uint4(0, 0, 0, 0);
  const int64_t pos = ks.w0 + (key0 + r - ks.n_c);
#pragma unroll
  for (int i = 0; i < WG::NC; ++i) {
    const int d0 = 8 * (c0 + kTPR * i);
    uint4 hi = keep_if(ok, R.v[i]);
    if (i == WG::NC - 1) {
      uint4 lo = z;
      if (ok && d0 >= rope0) rope8_hi_lo(R.v[i], pos, sm.rev, (d0 - rope0) >> 1, &hi, &lo);
      *reinterpret_cast<uint4*>(&sm.t.b.klo[r][d0 - (D - 64)]) = lo;
    }
    *reinterpret_cast<uint4*>(&sm.t.b.k[r][d0]) = hi;
  }
}

// ---------------------------------------------------------------- the query
// The QK dims of a block of S^T are shared by two waves (dq = 0, 1): steps [0, NSQ0) and
// [NSQ0, NS) of 16 dims, split so that both issue the same number of MFMAs (a step in the last 64
// dims carries a second product for the query remainder).
template <int D>
constexpr int qk_split() {
  constexpr int NS = D / 16, RS0 = (D - 64) / 16;
  const int total = NS + (NS - RS0);
  int acc = 0;
  for (int s = 0; s < NS; ++s) {
    acc += s >= RS0 ? 2 : 1;
    if (2 * acc >= total) return s + 1;
  }
  return NS;
}
template <int D, int DQ>
struct QkRange {
  static constexpr int NS = D / 16, RS0 = (D - 64) / 16, NSQ0 = qk_split<D>();
  static constexpr int S0 = DQ ? NSQ0 : 0, S1 = DQ ? NS : NSQ0;
  static constexpr int LO0 = S0 > RS0 ? S0 : RS0;        // first step with a query remainder
  static constexpr int NLO = S1 > LO0 ? S1 - LO0 : 0;    // steps with a query remainder
  static constexpr int NQ = S1 - S0, NLOA = NLO > 0 ? NLO : 1;
};

// The query's dims of this wave's steps, lane (head c, half u) holding dims 16 s + 8 u .. + 7 of
// head c; returns the lane's sum of squares of the raw values (query RMSNorm).
template <int D, int DQ>
__device__ __forceinline__ void load_query(const AttnArgs& a, int qi, int hq, uint4* q) {
  using R = QkRange<D, DQ>;
  const int ko = 8 * ((threadIdx.x & (kWave - 1)) >> 5);
  // heads past H (a partial block) compute with head H - 1's dims; their results are not written
  const uint16_t* src = a.q + ((int64_t)qi * a.H + min(hq, a.H - 1)) * D + ko;
#pragma unroll
  for (int s = R::S0; s < R::S1; ++s) q[s - R::S0] = *reinterpret_cast<const uint4*>(src + 16 * s);
}

// This lane's part of the query head's sum of squares (0 without the RMSNorm), once the loads
// have landed.
template <int D, int DQ>
__device__ __forceinline__ float query_sumsq(const AttnArgs& a, const uint4* q) {
  using R = QkRange<D, DQ>;
  float ss = 0.f;
  if (a.q_rms_eps > 0.f) {
#pragma unroll
    for (int s = R::S0; s < R::S1; ++s) {
      float f[8];
      unpack8(q[s - R::S0], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    }
  }
  return ss;
}

// The rotated dims among this wave's steps (the last d_rope of D): a bf16 value and a bf16
// remainder (qlo, indexed by step - LO0; zero elsewhere).
template <int D, int DQ>
__device__ __forceinline__ void rotate_query(const AttnArgs& a, const double* rev, int64_t t, uint4* q, uint4* qlo) {
  using R = QkRange<D, DQ>;
  const int ko = 8 * ((threadIdx.x & (kWave - 1)) >> 5);
  const int rope0 = D - a.d_rope;
#pragma unroll
  for (int s = R::LO0; s < R::S1; ++s) {
    uint4 lo = make_uint4(0, 0, 0, 0);
    const int d0 = 16 * s + ko;
    if (d0 >= rope0) rope8_hi_lo(q[s - R::S0], t, rev, (d0 - rope0) >> 1, &q[s - R::S0], &lo);
    qlo[s - R::LO0] = lo;
  }
}

// ---------------------------------------------------------------- S^T = K Q^T
// Partial S^T over this wave's steps for keys [32 kh, 32 kh + 32) of the staged tile and the
// wave's 32 heads; steps in the last 64 dims add the query remainders and, for window keys, the
// key remainders in klo. F8: the tile is a ring stage of fp8 codes (widened to bf16 as read).
template <int D, bool F8, bool WIN, int DQ>
__device__ __forceinline__ f32x16 tile_qk(const AttnSmem<D>& sm, int stage, const uint4* q, const uint4* qlo,
                                          int kh) {
  using R = QkRange<D, DQ>;
  const int lane = threadIdx.x & (kWave - 1);
  const int key = 32 * kh + (lane & 31), ko = 8 * (lane >> 5);
  constexpr int NP = 3;  // key operands in flight ahead of the MFMAs
  auto read = [&](int s) -> uint4 {
    if constexpr (F8) {
      const uint2 v = *reinterpret_cast<const uint2*>(&sm.t.r.k8[stage][s][key][ko]);
      return fp8x8_to_bf16(v.x, v.y);
    } else {
      return *reinterpret_cast<const uint4*>(&sm.t.b.k[key][16 * s + ko]);
    }
  };
  uint4 kv[NP];
#pragma unroll
  for (int u = 0; u < NP - 1; ++u)
    if (R::S0 + u < R::S1) kv[u] = read(R::S0 + u);
  f32x16 acc = {};
#pragma unroll
  for (int s = R::S0; s < R::S1; ++s) {
    const int j = s - R::S0;
    if (s + NP - 1 < R::S1) kv[(j + NP - 1) % NP] = read(s + NP - 1);
    acc = mfma32(kv[j % NP], q[j], acc);
    if (s >= R::LO0) {
      acc = mfma32(kv[j % NP], qlo[s - R::LO0], acc);
      if constexpr (WIN) {
        const uint4 kl = *reinterpret_cast<const uint4*>(&sm.t.b.klo[key][16 * (s - R::RS0) + ko]);
        acc = mfma32(kl, q[j], acc);
      }
    }
  }
  return acc;
}

// ---------------------------------------------------------------- S^T = K Q^T on the scaled FP4 MFMA
// MXFP4 entries (D a multiple of 64): v_mfma_scale_f32_32x32x64_f8f6f4 takes the stored e2m1 codes
// and E8M0 block exponents as they are. A operand: lane (key, g) holds the 32 dims of block 2s + g
// of its key (one 16-byte chunk of the row) with that block's exponent. B operand: lane (head, g)
// holds the query's dims 64s + 16g .. +15 in bytes 0-15 and 64s + 32 + 16g .. +15 in bytes 16-31
// as e4m3 codes, with one exponent per head and 64-dim step (the layout was checked on the GPU
// against a host product). The query enters as a sum of e4m3 parts, each scaled by 2^-4 of the
// previous one: two parts hold a bf16 value exactly (4 + 4 significant bits) unless it is below
// 2^-14 of its step's maximum; the last step (the rotated dims, d_rope <= 64, rotated in fp32)
// takes four parts, 16 significant bits, as many as the bf16 value plus remainder of the other
// path. Steps are split between the two dim halves so both issue the same number of MFMAs.
template <int D, int DQ>
struct F4Range {
  static constexpr int NK = D / 64;
  static constexpr int parts(int s) { return s == NK - 1 ? 4 : 2; }
  static constexpr int cut() {
    int total = 0, acc = 0;
    for (int s = 0; s < NK; ++s) total += parts(s);
    for (int s = 0; s < NK; ++s) {
      acc += parts(s);
      if (2 * acc >= total) return s + 1;
    }
    return NK;
  }
  static constexpr int S0 = DQ ? cut() : 0, S1 = DQ ? NK : cut();
  static constexpr int NKW = S1 > S0 ? S1 - S0 : 1;  // this wave's steps (1 when none, unused)
  static constexpr int count() {
    int n = 0;
    for (int s = S0; s < S1; ++s) n += parts(s);
    return n > 0 ? n : 1;
  }
  static constexpr int NP = count();  // this wave's query parts
};

// The query's dims of this wave's steps in the B layout above: 4 chunks of 8 bf16 per step.
template <int D, int DQ>
__device__ __forceinline__ void load_query_f4(const AttnArgs& a, int qi, int hq, uint4* qr) {
  using FR = F4Range<D, DQ>;
  const int g = (threadIdx.x & (kWave - 1)) >> 5;
  const uint16_t* src = a.q + ((int64_t)qi * a.H + min(hq, a.H - 1)) * D;
#pragma unroll
  for (int s = FR::S0; s < FR::S1; ++s) {
    const int j = 4 * (s - FR::S0);
    qr[j + 0] = *reinterpret_cast<const uint4*>(src + 64 * s + 16 * g);
    qr[j + 1] = *reinterpret_cast<const uint4*>(src + 64 * s + 16 * g + 8);
    qr[j + 2] = *reinterpret_cast<const uint4*>(src + 64 * s + 32 + 16 * g);
    qr[j + 3] = *reinterpret_cast<const uint4*>(src + 64 * s + 32 + 16 * g + 8);
  }
}

// Eight consecutive dims (RoPE pairs pair0 .. pair0 + 3) rotated to position pos, in fp32.
__device__ __forceinline__ void rope8_f32(float* f, int64_t pos, const double* rev, int pair0) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float cs, sn;
    rope_cs(rev[pair0 + p], pos, &cs, &sn);
    const float u0 = f[2 * p], u1 = f[2 * p + 1];
    f[2 * p] = u0 * cs - u1 * sn;
    f[2 * p + 1] = u0 * sn + u1 * cs;
  }
}

// LDS exchange of the query parts between the two waves of a (head half, dim half) pair, in the
// tile region (free until the first tile is staged).
template <int D>
struct F4Xchg {
  static constexpr int NPMAX = F4Range<D, 0>::NP > F4Range<D, 1>::NP ? F4Range<D, 0>::NP : F4Range<D, 1>::NP;
  int part[2][2][NPMAX][kWave][8];  // [dq][hh][part][lane]
  int exp[2][2][D / 64][kWave];     // [dq][hh][step][lane]
  float ss[2][2][2][32];            // [dq][hh][kh][head]: sums of squares of each wave's steps
};

// The query as e4m3 parts (qf, B operands in step order) with one exponent per step (qe: part p
// of step s is scaled by 2^(qe - 4p)). The two waves of a (head half, dim half) pair share the
// work: wave kh converts the steps j = s - S0 with j % 2 == kh and the two swap results through
// LDS (one barrier). Two-part steps (raw bf16 dims) split each value by truncation: the top 4
// significant bits and the exact remainder; the last step's rotated dims (fp32) take four parts,
// each the rounding of the previous remainder. Every rotated or normal-range value is held
// exactly (to 16 significant bits when rotated); a raw value below 2^-13 of its step's maximum
// may round in the e4m3 subnormal range, an error under 2^-17 of that maximum. Writes the query's
// sums of squares per dim half (RMSNorm) to qss. Where the exchange does not fit the tile region
// (small D), each wave converts all of its steps.
template <int D, int DQ>
__device__ __forceinline__ void quantize_query_f4(const AttnArgs& a, AttnSmem<D>& sm, int64_t t, const uint4* qr,
                                                  int hh, int kh, i32x8* qf, int* qe) {
  using FR = F4Range<D, DQ>;
  constexpr bool SHARE = sizeof(F4Xchg<D>) <= sizeof(sm.t);
  F4Xchg<D>& X = *reinterpret_cast<F4Xchg<D>*>(&sm.t);
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 5;
  const int rope0 = D - a.d_rope;
  const bool rms = a.q_rms_eps > 0.f;
  float ss = 0.f;
  int pb = 0;  // first part of step s
#pragma unroll
  for (int s = FR::S0; s < FR::S1; ++s) {
    const int j = s - FR::S0;
    if (!SHARE || (j & 1) == kh) {
      float x[32];
#pragma unroll
      for (int c = 0; c < 4; ++c) unpack8(qr[4 * j + c], x + 8 * c);
      if (rms) {
#pragma unroll
        for (int e = 0; e < 32; ++e) ss += x[e] * x[e];
      }
      if (s == FR::NK - 1) {  // the rotated dims (d_rope <= 64) all lie in the last step
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int d0 = 64 * s + (c < 2 ? 16 * g + 8 * c : 32 + 16 * g + 8 * (c - 2));
          if (d0 >= rope0) rope8_f32(x + 8 * c, t, sm.rev, (d0 - rope0) >> 1);
        }
      }
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
      amax = max_xor32(amax);  // the head's 64 dims of the step
      const int E = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 8 : 0;  // amax * 2^-E in [128, 256)
      qe[j] = E;
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = __builtin_amdgcn_ldexpf(x[e], -E);
      if (FR::parts(s) == 2) {
        i32x8 hi, lo;
#pragma unroll
        for (int wd = 0; wd < 8; ++wd) {
          float h[4], l[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[e] = __uint_as_float(__float_as_uint(x[4 * wd + e]) & 0xFFF00000u);  // 4 significant bits
            l[e] = (x[4 * wd + e] - h[e]) * 16.f;                                  // the exact rest
          }
          int wh = __builtin_amdgcn_cvt_pk_fp8_f32(h[0], h[1], 0, false);
          hi[wd] = __builtin_amdgcn_cvt_pk_fp8_f32(h[2], h[3], wh, true);
          int wl = __builtin_amdgcn_cvt_pk_fp8_f32(l[0], l[1], 0, false);
          lo[wd] = __builtin_amdgcn_cvt_pk_fp8_f32(l[2], l[3], wl, true);
        }
        qf[pb] = hi;
        qf[pb + 1] = lo;
      } else {
#pragma unroll
        for (int p = 0; p < FR::parts(s); ++p) {
          i32x8 v;
#pragma unroll
          for (int wd = 0; wd < 8; ++wd) {
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * wd], x[4 * wd + 1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * wd + 2], x[4 * wd + 3], word, true);
            v[wd] = word;
            if (p + 1 < FR::parts(s)) {  // the remainder (exact: within 2^-4 of the value), scaled up
              const auto lo2 = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
              const auto hi2 = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
              x[4 * wd] = (x[4 * wd] - lo2[0]) * 16.f;
              x[4 * wd + 1] = (x[4 * wd + 1] - lo2[1]) * 16.f;
              x[4 * wd + 2] = (x[4 * wd + 2] - hi2[0]) * 16.f;
              x[4 * wd + 3] = (x[4 * wd + 3] - hi2[1]) * 16.f;
            }
          }
          qf[pb + p] = v;
        }
      }
      if constexpr (SHARE) {
#pragma unroll
        for (int p = 0; p < FR::parts(s); ++p)
#pragma unroll
          for (int wd = 0; wd < 8; ++wd) X.part[DQ][hh][pb + p][lane][wd] = qf[pb + p][wd];
        X.exp[DQ][hh][s][lane] = E;
      }
    }
    pb += FR::parts(s);
  }
  ss = add_xor32(ss);
  if constexpr (!SHARE) {
    if (kh == 0 && lane < 32) sm.qss[DQ][32 * hh + lane] = ss;
    return;
  }
  if (lane < 32) X.ss[DQ][hh][kh][lane] = ss;
  __syncthreads();
  pb = 0;
#pragma unroll
  for (int s = FR::S0; s < FR::S1; ++s) {
    const int j = s - FR::S0;
    if ((j & 1) != kh) {
#pragma unroll
      for (int p = 0; p < FR::parts(s); ++p)
#pragma unroll
        for (int wd = 0; wd < 8; ++wd) qf[pb + p][wd] = X.part[DQ][hh][pb + p][lane][wd];
      qe[j] = X.exp[DQ][hh][s][lane];
    }
    pb += FR::parts(s);
  }
  if (kh == 0 && lane < 32) sm.qss[DQ][32 * hh + lane] = X.ss[DQ][hh][0][lane] + X.ss[DQ][hh][1][lane];
}

// Partial S^T over this wave's steps for keys [32 kh, 32 kh + 32) of the staged MXFP4 tile.
template <int D, int DQ>
__device__ __forceinline__ f32x16 tile_qk_f4(const AttnSmem<D>& sm, const i32x8* qf, const int* qe, int kh) {
  using FR = F4Range<D, DQ>;
  const int lane = threadIdx.x & (kWave - 1);
  const int key = 32 * kh + (lane & 31), g = lane >> 5;
  f32x16 acc = {};
  int pi = 0;
#pragma unroll
  for (int s = FR::S0; s < FR::S1; ++s) {
    const uint4 kc = *reinterpret_cast<const uint4*>(&sm.t.b.k4[2 * s + g][key][0]);
    const int ka = sm.t.b.s4[key][2 * s + g];
    const i32x8 av = {(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < FR::parts(s); ++p)
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qf[pi++], acc, 4, 0, 0, ka, 0,
                                                            qe[s - FR::S0] - 4 * p + 127);
  }
  return acc;
}

// ---------------------------------------------------------------- softmax
// Per-lane online-softmax state of the lane's head. m is the exponent base of the running sums;
// it may lag the true running maximum by up to kRescaleSlack (p <= 2^8), so O is rescaled only
// when a logit exceeds it by more than that. l holds the keys this lane wrote P for.
template <int NO>
struct HeadState {
  f32x16 o[NO];  // O^T rows (value dims) of this wave's blocks, column = the lane's head
  float m, l;
};

// Softmax of one staged tile. The two waves of a block of S^T (first and second half of the dims)
// hand each other the half of their partial logits that the other needs through LDS; each then
// forms the logits of half of the block's keys (valid: the tile's key mask; vsc: per-key scales of
// fp8 entries, else 1), writes their P^T with the current exponent base and flags the tile if a
// logit exceeds its head's base by more than the slack. After the barrier that makes P^T visible,
// a flagged tile (the first one, and rarely another) takes the base from the four waves' maxima:
// every wave rescales its O and l and forms its P^T again. Ends with P^T visible.
template <int D, int NO>
__device__ __forceinline__ void tile_softmax(const AttnArgs& a, AttnSmem<D>& sm, HeadState<NO>& st, const f32x16& s,
                                             int w, uint64_t valid, const float* vsc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int hh = w & 1, kh = (w >> 1) & 1, dq = w >> 2;
  const int hl = 32 * hh + (lane & 31), kr = 32 * kh + 4 * (lane >> 5);  // keys kr + 8 g + e
  // the partner's groups of this wave's partial logits
#pragma unroll
  for (int gg = 0; gg < 2; ++gg) {
    const int g = 2 * (1 - dq) + gg;
    sm.xs[w][gg][lane] = f32x4{s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]};
  }
  __syncthreads();
  const float qs = a.q_rms_eps > 0.f ? 1.0f / sqrtf((sm.qss[0][hl] + sm.qss[1][hl]) / (float)D + a.q_rms_eps)
                                     : 1.0f;  // query RMSNorm factor of the lane's head
  float lt = 0.f;
  // logits of this wave's keys (own partial + the partner's, added in dims order), then P^T with
  // exponent base `base`; returns the head's maximum over this wave's keys
  auto form_p = [&](float base) {
    float mloc = -INFINITY;
    lt = 0.f;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g = 2 * dq + gg;
      const f32x4 o = sm.xs[w ^ 4][gg][lane];
      const f32x4 vk = vsc ? *reinterpret_cast<const f32x4*>(vsc + kr + 8 * g) : f32x4{1.f, 1.f, 1.f, 1.f};
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kr + 8 * g + e;
        const float sum = dq == 0 ? s[4 * g + e] + o[e] : o[e] + s[4 * g + e];
        const bool ok = (valid >> key) & 1;
        const float x = ok ? sum * (qs * a.scale_log2 * vk[e]) : -INFINITY;
        mloc = fmaxf(mloc, x);
        // exponent <= kRescaleSlack once the base is set; below the fp32 range p flushes to 0
        const float p = __builtin_amdgcn_exp2f(x - base);
        lt += p;
        pv[e] = ok ? p * vk[e] : 0.f;  // value-side scale folded into P
      }
      uint2 wv;
      wv.x = cvt_bf16x2(pv[0], pv[1]);
      wv.y = cvt_bf16x2(pv[2], pv[3]);
      *reinterpret_cast<uint2*>(&sm.p[hl][kr + 8 * g]) = wv;
    }
    return max_xor32(mloc);
  };
  {
    const float mloc = form_p(st.m == -INFINITY ? 0.f : st.m);
    if (lane < 32) sm.xmax[2 * kh + dq][hl] = mloc;
    if (__ballot(mloc > st.m + kRescaleSlack) && lane == 0) sm.rescale = 1;
  }
  __syncthreads();
  if (sm.rescale) {  // the same in every wave: move the exponent base up, rescale O and l
    const float tmax = fmaxf(fmaxf(sm.xmax[0][hl], sm.xmax[1][hl]), fmaxf(sm.xmax[2][hl], sm.xmax[3][hl]));
    if (tmax > st.m + kRescaleSlack) {
      const float alpha = st.m == -INFINITY ? 0.f : exp2f(st.m - tmax);
      st.l *= alpha;
      st.m = tmax;
#pragma unroll
      for (int n = 0; n < NO; ++n) st.o[n] *= alpha;
    }
    form_p(st.m);
    __syncthreads();
    if (threadIdx.x == 0) sm.rescale = 0;  // read by every wave before the barrier above
  }
  st.l += lt;
}

// ---------------------------------------------------------------- O^T += V^T P^T
// Over the staged tile (four steps of 16 keys) for this wave's value-dim blocks. V^T (A operand):
// lane (dim c, half u) holds keys 8u .. 8u+7 of the step for its dim: one transposed byte read of
// an fp8 ring stage (keys the mask `valid` hides are zeroed: a ring row may hold anything), or two
// transposed 16-bit reads of 4 keys from a bf16 tile; P^T (B operand): lane (head c, half u) the
// same keys of its head.
template <int D, int NO, int NB, bool F8>
__device__ __forceinline__ void tile_pv(const AttnSmem<D>& sm, HeadState<NO>& st, int hh, int vq, int stage,
                                        uint64_t valid) {
  const int lane = threadIdx.x & (kWave - 1);
  const int hl = 32 * hh + (lane & 31), u = lane >> 5, L = lane & 15;
  const bool all = valid == ~0ull;
#pragma unroll
  for (int ks = 0; ks < kTK / 16; ++ks) {
    const uint4 pb = *reinterpret_cast<const uint4*>(&sm.p[hl][16 * ks + 8 * u]);
    uint32_t m0 = ~0u, m1 = ~0u;  // byte masks of the lane's 8 keys
    if (F8 && !all) {
      const uint32_t bits = (uint32_t)(valid >> (16 * ks + 8 * u)) & 0xFFu;
      m0 = m1 = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m0 |= ((bits >> i) & 1u) ? (0xFFu << (8 * i)) : 0u;
        m1 |= ((bits >> (4 + i)) & 1u) ? (0xFFu << (8 * i)) : 0u;
      }
    }
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      const int b = vq * NO + n;
      if (NB % 4 != 0 && b >= NB) continue;
      uint4 va;
      if constexpr (F8) {
        const int key0 = 16 * ks + 8 * u + (L >> 1);
        const int ch = 2 * b + ((lane >> 4) & 1);  // dims 16 ch .. 16 ch + 15
        const i32x2 v =
            __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(&sm.t.r.k8[stage][ch][key0][8 * (L & 1)]));
        va = fp8x8_to_bf16((uint32_t)v.x & m0, (uint32_t)v.y & m1);
      } else {
        const int key0 = 16 * ks + 8 * u + (L >> 2);
        const int dim0 = 32 * b + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&sm.t.b.k[key0][dim0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&sm.t.b.k[key0 + 4][dim0]));
        va = __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      st.o[n] = mfma32(va, pb, st.o[n]);
    }
  }
}

// ---------------------------------------------------------------- the kernel
// The work of one wave: DQ is the wave's half of the QK dims (a template parameter, so that only
// that half's query registers exist). F4 (MXFP4 entries, D a multiple of 64): the entry keys go
// through the scaled FP4 MFMA with the query as e4m3 parts; the bf16 query (window keys) is then
// loaded after the entries, so the two register sets are never live together.
template <int D, int DV, int KV, int DQ, bool F4>
__device__ __forceinline__ void attn_body(const AttnArgs& a, AttnSmem<D>& sm) {
  static_assert(!F4 || (KV == kKvMxfp4 && D % 64 == 0), "FP4 QK needs MXFP4 entries and D % 64 == 0");
  using R = QkRange<D, DQ>;
  constexpr int NB = DV / 32, NO = (NB + 3) / 4;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = wave_id();
  // QK: wave (hh, kh, dq) = head half, key half, half of the dims; PV: (hh, vq) = head half,
  // quarter of the value dims; w = hh + 2 kh + 4 dq = hh + 2 vq
  const int hh = w & 1, kh = (w >> 1) & 1, vq = w >> 1;
  const int hl = 32 * hh + (lane & 31);
  const int split = (int)(blockIdx.x % (unsigned)a.n_splits);
  const int qh = (int)(blockIdx.x / (unsigned)a.n_splits);
  const int qi = qh / a.n_hb;
  const int hq = (qh % a.n_hb) * kHB + hl;  // this lane's head

  constexpr bool F8 = KV == kKvFp8;
  using FR = F4Range<D, DQ>;
  const bool dense = a.topk == nullptr;
  // the query's dims of this lane's head and wave's steps, then the query's position and entry
  // count (their latency overlaps the listing of the split's rows)
  uint4 q[R::NQ], qlo[R::NLOA];
  uint4 qr[F4 ? 4 * FR::NKW : 1];
  if constexpr (F4)
    load_query_f4<D, DQ>(a, qi, hq, qr);
  else
    load_query<D, DQ>(a, qi, hq, q);
  const KeySpace ks = key_space(a, qi);

  int key_begin, key_end;
  if (a.n_esplits < a.n_splits) {  // entry splits, then window splits
    if (split < a.n_esplits) {
      key_begin = split * a.keys_per_split;
      key_end = min(ks.n_c, key_begin + a.keys_per_split);
    } else {
      key_begin = ks.n_c + (split - a.n_esplits) * a.win_per_split;
      key_end = min(ks.n_c + ks.n_w, key_begin + a.win_per_split);
    }
  } else {
    key_begin = split * a.keys_per_split;
    key_end = min(ks.n_c + ks.n_w, key_begin + a.keys_per_split);
  }
  const int e_end = min(key_end, ks.n_c);  // entry keys [key_begin, e_end), window keys after
  const int w_begin = max(key_begin, ks.n_c);
  const int n_et = key_begin < e_end ? (e_end - key_begin + kTK - 1) / kTK : 0;  // entry tiles
  const int64_t seq = (int64_t)(a.ckv_seq ? qi / a.q_per_seq : 0) * a.ckv_seq;
  constexpr int row_bytes = KV == kKvBf16 ? 2 * D : (KV == kKvFp8 ? D : D / 2);
  constexpr int srow_bytes = KV == kKvFp8 ? 4 : (KV == kKvMxfp4 ? D / 32 : 0);
  const uint8_t* cbase = reinterpret_cast<const uint8_t*>(a.ckv) + seq * row_bytes;
  const uint8_t* sbase = a.ckv_scale ? reinterpret_cast<const uint8_t*>(a.ckv_scale) + seq * srow_bytes : nullptr;
  // dense fp8 entries: the first tile's rows are known now (entry = key)
  if (F8 && dense && n_et > 0)
    issue_tile_f8<D>(sm, 0, cbase, reinterpret_cast<const float*>(sbase), key_begin, e_end, key_begin, true);
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
    if (a.x_new && j == 0 && split == 0 && qh % a.n_hb == 0)
      append_new_tokens(a.x_new, a.z_new, a.ring_w, a.ring_z, qi, a.q_per_seq, ks.t, a.ring_cap, a.D, tid, kNT);
  }
  // the RoPE table in revolutions per position, base^(-2i / d_rope) / (2 pi), in fp64
  // (pair i: rope_step^i / (2 pi), the power formed by squaring, a few fp64 roundings)
  if (w == 0 && 2 * lane < a.d_rope) {
    double f = 0.15915494309189533576888376337251, r = a.rope_step;
#pragma unroll
    for (int b = 0; b < 5; ++b) {  // lane < 32
      if ((lane >> b) & 1) f *= r;
      r *= r;
    }
    sm.rev[lane] = f;
  }
  if (tid == 0) sm.rescale = 0;
  __syncthreads();  // sidx and the RoPE table ready

  // every load so far (the query, the row lists, a dense first tile) has landed: the loop then
  // waits on tile loads only where a tile is used, never because a query register might be
  // pending
  __builtin_amdgcn_s_waitcnt(0);
  if (F8 && !dense && n_et > 0)
    issue_tile_f8<D>(sm, 0, cbase, reinterpret_cast<const float*>(sbase), key_begin, e_end, key_begin, false);
  i32x8 qf[F4 ? FR::NP : 1];
  int qe[F4 ? FR::NKW : 1];
  if constexpr (F4) {
    quantize_query_f4<D, DQ>(a, sm, ks.t, qr, hh, kh, qf, qe);  // qss too; one barrier
  } else {
    float ss = query_sumsq<D, DQ>(a, q);
    rotate_query<D, DQ>(a, sm.rev, ks.t, q, qlo);
    ss = add_xor32(ss);
    if (kh == 0 && lane < 32) sm.qss[DQ][hl] = ss;  // read after the first tile's barriers
  }
  if (F8 && n_et > 1)
    issue_tile_f8<D>(sm, 1, cbase, reinterpret_cast<const float*>(sbase), key_begin + kTK, e_end, key_begin, dense);

  HeadState<NO> st;
#pragma unroll
  for (int n = 0; n < NO; ++n) st.o[n] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;

  // phase 1: compressed entries
  for (int t = 0; t < n_et; ++t) {
    const int key0 = key_begin + kTK * t;
    int stage = 0;
    const float* vsc = nullptr;
    if constexpr (F8) {
      stage = t % kStages;
      wait_tile_f8<D>(t + 1 < n_et);  // this wave's requests of tile t have landed
      __syncthreads();                // everyone's have; the previous tile's reads are done
      vsc = &sm.t.r.sc[stage][0];
    } else {
      TileRegs<D, KV> RT;
      entry_load<D, KV>(cbase, sbase, key0, e_end, key_begin, sm, RT);
      __syncthreads();  // the previous tile's reads are done
      entry_store<D, KV, F4>(sm, RT, DV);
      __syncthreads();
    }
    const uint64_t valid = tile_mask<D>(sm, key0, e_end, key_begin);
    f32x16 s;
    if constexpr (F4)
      s = tile_qk_f4<D, DQ>(sm, qf, qe, kh);
    else
      s = tile_qk<D, F8, false, DQ>(sm, stage, q, qlo, kh);
    tile_softmax<D, NO>(a, sm, st, s, w, valid, vsc);
    if (F8 && t + 2 < n_et)  // ring stage (t + 2) % 3 was last read by tile t - 1, finished by all
      issue_tile_f8<D>(sm, (t + 2) % kStages, cbase, reinterpret_cast<const float*>(sbase), key0 + 2 * kTK, e_end,
                       key_begin, dense);
    tile_pv<D, NO, NB, F8>(sm, st, hh, vq, stage, valid);
  }
  // phase 2: window tokens (the bf16 tile overlays the ring: staged after the last entry tile's reads)
  if constexpr (F4) {
    if (w_begin < key_end) {  // the bf16 query for the window keys
      load_query<D, DQ>(a, qi, hq, q);
      rotate_query<D, DQ>(a, sm.rev, ks.t, q, qlo);
    }
  }
  for (int key0 = w_begin; key0 < key_end; key0 += kTK) {
    WinRegs<D> RW;
    window_load<D>(a, key0, key_end, key_begin, sm, RW);
    __syncthreads();
    window_store<D>(a, ks, key0, sm, RW);
    __syncthreads();
    const uint64_t valid = tile_mask<D>(sm, key0, key_end, key_begin);
    const f32x16 s = tile_qk<D, false, true, DQ>(sm, 0, q, qlo, kh);
    tile_softmax<D, NO>(a, sm, st, s, w, valid, nullptr);
    tile_pv<D, NO, NB, false>(sm, st, hh, vq, 0, valid);
  }

  // the head's key sum: over the lane halves, then over the four waves that wrote its P
  {
    const float lw = add_xor32(st.l);
    if (lane < 32) sm.lsum[2 * kh + DQ][hl] = lw;
  }
  __syncthreads();
  const float lt = sm.lsum[0][hl] + sm.lsum[1][hl] + sm.lsum[2][hl] + sm.lsum[3][hl];
  const int u4 = 4 * (lane >> 5);  // O^T rows of this lane: 32 b + 8 g + u4 + e

  if (a.n_splits == 1) {
    if (hq >= a.H) return;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* dst = a.out + ((int64_t)qi * a.H + hq) * DV;
#pragma unroll
    for (int n = 0; n < NO; ++n) {
      const int b = vq * NO + n;
      if (NB % 4 != 0 && b >= NB) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 pk;
        pk.x = cvt_bf16x2(st.o[n][4 * g] * inv, st.o[n][4 * g + 1] * inv);
        pk.y = cvt_bf16x2(st.o[n][4 * g + 2] * inv, st.o[n][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(dst + 32 * b + 8 * g + u4) = pk;
      }
    }
    if (a.out_lse && vq == 0 && lane < 32)
      a.out_lse[(int64_t)qi * a.H + hq] = lt > 0.f ? (st.m + log2f(lt)) * kLn2 : -INFINITY;
    return;
  }

  // split partial: O / l in fp16 (a convex combination of value rows, so within their range; the
  // relative rounding 2^-11 sits well below the output's bf16 rounding), exponent base and sum
  const int64_t prow = (((int64_t)qh * a.n_splits + split) * kHB + hl);
  uint16_t* dst = a.part_o + prow * DV;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int n = 0; n < NO; ++n) {
    const int b = vq * NO + n;
    if (NB % 4 != 0 && b >= NB) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 pk;
      pk.x = cvt_f16x2(st.o[n][4 * g] * inv, st.o[n][4 * g + 1] * inv);
      pk.y = cvt_f16x2(st.o[n][4 * g + 2] * inv, st.o[n][4 * g + 3] * inv);
      *reinterpret_cast<uint2*>(dst + 32 * b + 8 * g + u4) = pk;
    }
  }
  if (vq == 0 && lane < 32) {
    a.part_ml[prow * 2 + 0] = st.m;
    a.part_ml[prow * 2 + 1] = lt;
  }
}

template <int D, int DV, int KV, bool F4>
__global__ __launch_bounds__(kNT, 1) void attn_kernel(AttnArgs a) {
  __shared__ AttnSmem<D> sm;
  if (wave_id() >> 2)
    attn_body<D, DV, KV, 1, F4>(a, sm);
  else
    attn_body<D, DV, KV, 0, F4>(a, sm);
}

// One workgroup per (query, head): log-sum-exp merge of the split partials, split s weighted by
// 2^(m_s - M) l_s. Thread t owns dims 4t..4t+3 (d_v <= 4 * kMergeNT). Split rows are read
// kMergeBatch at a time, the batch requested before the previous one is summed; rows past the
// last split repeat it with weight 0, so every load is unconditional.
constexpr int kMergeNT = 128;
constexpr int kMergeBatch = 8;
__global__ __launch_bounds__(kMergeNT) void attn_merge_kernel(AttnArgs a) {
  __shared__ float wsh[kMaxSplits + kMergeBatch];
  __shared__ float red[2];
  const int qi = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int S = a.n_splits;
  const int64_t row0 = ((int64_t)(qi * a.n_hb + h / kHB) * S) * kHB + h % kHB;  // split s: row0 + s * kHB
  const int dd = min(4 * tid, a.d_v - 4);  // threads past d_v read the last dims and store nothing
  if (tid < kWave) {
    float mx = -INFINITY;
    for (int sp = tid; sp < S; sp += kWave) mx = fmaxf(mx, a.part_ml[(row0 + (int64_t)sp * kHB) * 2]);
    mx = wave_max(mx);
    const float Mb = mx == -INFINITY ? 0.f : mx;
    float l = 0.f;
    for (int sp = tid; sp < S + kMergeBatch; sp += kWave) {
      float wt = 0.f;
      if (sp < S) {
        const float2 ml = *reinterpret_cast<const float2*>(&a.part_ml[(row0 + (int64_t)sp * kHB) * 2]);
        wt = exp2f(ml.x - Mb) * ml.y;
        l += wt;
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
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  auto fetch = [&](uint2 (&v)[kMergeBatch], int s0) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      v[u] = *reinterpret_cast<const uint2*>(a.part_o + (row0 + (int64_t)min(s0 + u, S - 1) * kHB) * a.d_v + dd);
  };
  auto sum = [&](const uint2 (&v)[kMergeBatch], int s0) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const f16x4 h = __builtin_bit_cast(f16x4, v[u]);
      acc += wsh[s0 + u] * f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    }
  };
  uint2 v0[kMergeBatch], v1[kMergeBatch];
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
  int n_hb, n_splits, n_esplits, keys_per_split, win_per_split;
  size_t ws;  // bytes of the split partials
};

// Splits of a query's key set (at most kMaxSplits, each a whole number of 64-key tiles of at most
// kMaxSplitKeys keys). Either the keys are cut in order (entries, then window tokens), or the
// entries are cut into splits and each window tile gets a split of its own. With one workgroup
// per CU a launch takes ceil(workgroups / kCUs) rounds of its longest split and a workgroup's
// fixed prologue and epilogue, plus the merge launch when the keys are split (with a CU budget
// below the GPU's 256, for calls that share the GPU with kernels of another stream, the rounds
// are counted over that many CUs, so fewer, longer splits win); a window tile
// (loaded and rotated when staged) counts one and a half entry tiles. The cheapest plan wins
// (ties: the first found, fewer splits).
static int g_attn_cus = kCUs;  // CUs a split plan of the 64-head kernel counts on

static AttnPlan plan_attn(int nq, int H, int d_v, int max_entries, int W) {
  AttnPlan p{};
  const int cus = g_attn_cus;
  p.n_hb = (H + kHB - 1) / kHB;
  const int64_t base = (int64_t)nq * p.n_hb;
  const int te = (max(max_entries, 0) + kTK - 1) / kTK, tw = (max(W, 0) + kTK - 1) / kTK;
  const int tiles = max(te + tw, 1);
  auto rounds = [&](int s) { return (base * s + cus - 1) / cus; };
  int64_t best_cost = -1;
  // keys in order: the split holding the window tiles is the longest
  for (int s = 1; s <= kMaxSplits && s <= tiles; ++s) {
    const int per = (tiles + s - 1) / s;
    if ((tiles + per - 1) / per != s || per * kTK > kMaxSplitKeys) continue;
    const int64_t cost = rounds(s) * (2 * per + min(tw, per) + 2 * kWgFixedTiles) + (s > 1 ? 2 * kMergeTiles : 0);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      p.n_splits = p.n_esplits = s;
      p.keys_per_split = per * kTK;
    }
  }
  // entry splits plus one split per window tile
  if (te > 0 && tw > 0) {
    for (int se = 1; se + tw <= kMaxSplits && se <= te; ++se) {
      const int per = (te + se - 1) / se;
      if ((te + per - 1) / per != se || per * kTK > kMaxSplitKeys) continue;
      const int64_t cost = rounds(se + tw) * (max(2 * per, 3) + 2 * kWgFixedTiles) + 2 * kMergeTiles;
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        p.n_splits = se + tw;
        p.n_esplits = se;
        p.keys_per_split = per * kTK;
        p.win_per_split = kTK;
      }
    }
  }
  if (best_cost < 0) {  // refused by launch_attn: more than kMaxSplits splits of kMaxSplitKeys keys
    p.n_splits = p.n_esplits = kMaxSplits + 1;
    p.keys_per_split = kMaxSplitKeys;
  }
  p.ws = p.n_splits > 1 ? (size_t)base * p.n_splits * kHB * (2 * (size_t)d_v + 2 * sizeof(float)) : 0;
  return p;
}

typedef void (*AttnKernel)(AttnArgs);

template <int KV, bool F4 = false>
static AttnKernel pick_dims(int D, int d_v) {
  if (D == 576 && d_v == 512) return attn_kernel<576, 512, KV, F4>;
  if (D == 128 && d_v == 128) return attn_kernel<128, 128, KV, F4>;
  if (D == 64 && d_v == 32) return attn_kernel<64, 32, KV, F4>;
  if (D == 256 && d_v == 128) return attn_kernel<256, 128, KV, F4>;
  return nullptr;
}

// Compiled (D, d_v) pairs (every D a multiple of 64, so each has the FP4-QK variant).
static AttnKernel pick_kernel(int D, int d_v, int kv, bool qk_fp4 = false) {
  if (kv == kKvMxfp4) return qk_fp4 ? pick_dims<kKvMxfp4, true>(D, d_v) : pick_dims<kKvMxfp4>(D, d_v);
  return kv == kKvFp8 ? pick_dims<kKvFp8>(D, d_v) : pick_dims<kKvBf16>(D, d_v);
}

static int check_common(const char* name, int H, int D, int d_rope, int d_v, int W, int ckv_dtype, float q_rms_eps) {
  CSKV_REQUIRE(H >= 1 && H <= 128, CSKV_EINVAL, "%s: H=%d outside [1, 128]", name, H);
  CSKV_REQUIRE(D % 32 == 0 && D >= 32, CSKV_EINVAL, "%s: D=%d must be a positive multiple of 32", name, D);
  CSKV_REQUIRE(d_v % 16 == 0 && d_v >= 16 && d_v <= D, CSKV_EINVAL, "%s: d_v=%d", name, d_v);
  CSKV_REQUIRE(d_rope >= 0 && d_rope % 8 == 0 && d_rope <= D, CSKV_EINVAL, "%s: d_rope=%d", name, d_rope);
  CSKV_REQUIRE(W >= 0, CSKV_EINVAL, "%s: W=%d", name, W);
  CSKV_REQUIRE(q_rms_eps >= 0.f && q_rms_eps < INFINITY, CSKV_EINVAL, "%s: q_rms_eps=%g", name, (double)q_rms_eps);
  CSKV_REQUIRE(d_rope <= 2 * kMaxRopePairs, CSKV_ENOTSUP, "%s: d_rope=%d > %d", name, d_rope, 2 * kMaxRopePairs);
  const int kv = ckv_dtype & ~CSKV_QK_FP4;
  CSKV_REQUIRE(kv == CSKV_BF16 || kv == CSKV_FP8_E4M3 || kv == CSKV_MXFP4, CSKV_EINVAL, "%s: ckv_dtype=%d", name,
               ckv_dtype);
  CSKV_REQUIRE(!(ckv_dtype & CSKV_QK_FP4) || (kv == CSKV_MXFP4 && D % 64 == 0), CSKV_EINVAL,
               "%s: CSKV_QK_FP4 needs CSKV_MXFP4 entries and D %% 64 == 0 (D=%d)", name, D);
  CSKV_REQUIRE(pick_kernel(D, d_v, kKvBf16) != nullptr, CSKV_ENOTSUP,
               "%s: (D, d_v) = (%d, %d) not compiled (576/512, 128/128, 256/128, 64/32)", name, D, d_v);
  return CSKV_OK;
}

static int launch_attn(const char* name, AttnArgs a, const AttnPlan& p, bool qk_fp4, void* ws, size_t ws_bytes,
                       hipStream_t s) {
  CSKV_REQUIRE(p.ws == 0 || (ws && ws_bytes >= p.ws), CSKV_EWORKSPACE, "%s: workspace %zu < %zu bytes", name,
               ws_bytes, p.ws);
  a.n_hb = p.n_hb;
  a.n_splits = p.n_splits;
  a.keys_per_split = p.keys_per_split;
  a.n_esplits = p.n_esplits;
  a.win_per_split = p.win_per_split;
  CSKV_REQUIRE(p.n_splits <= kMaxSplits, CSKV_ENOTSUP, "%s: %d key splits > %d (key set too large)", name,
               p.n_splits, kMaxSplits);
  CSKV_REQUIRE(p.n_splits == 1 || a.d_v <= 4 * kMergeNT, CSKV_ENOTSUP, "%s: d_v=%d > %d with split keys", name,
               a.d_v, 4 * kMergeNT);
  if (p.n_splits > 1) {
    a.part_o = reinterpret_cast<uint16_t*>(ws);
    a.part_ml = reinterpret_cast<float*>(a.part_o + (size_t)a.nq * p.n_hb * p.n_splits * kHB * a.d_v);
  }
  const int64_t total = (int64_t)a.nq * p.n_hb * p.n_splits;
  CSKV_REQUIRE(total < (1ll << 31), CSKV_ENOTSUP, "%s: %lld workgroups", name, (long long)total);
  AttnKernel kern = pick_kernel(a.D, a.d_v, a.kv_dtype, qk_fp4);
  hipLaunchKernelGGL(kern, dim3((unsigned)total), dim3(kNT), 0, s, a);
  CSKV_LAUNCH_CHECK(name);
  if (p.n_splits > 1) {
    hipLaunchKernelGGL(attn_merge_kernel, dim3(a.nq, a.H), dim3(kMergeNT), 0, s, a);
    CSKV_LAUNCH_CHECK(name);
  }
  return CSKV_OK;
}

}  // namespace cskv

namespace cskv {

static int g_attn_path = 0;  // 0: by the call's shape; 1: the 64-head kernel; 2: the 16-head kernel

// The 16-head kernel takes short key sets of few queries: a workgroup's prologue then lasts as
// long as its tiles, and its two workgroups per CU hide one another's. The 64-head kernel takes
// everything else. Measured crossover (cold calls, 64 heads, D = 512+64, fp8 and bf16 entries):
// the 16-head kernel is faster up to about 4096 (query, key) pairs per call — 16 queries of
// 192 or 256 keys, 8 of 512 — and slower beyond (at 32 queries of 256 keys, 31.5 µs against
// 26.6 µs).
static bool use_g16(int nq, int max_keys) {
  if (g_attn_path) return g_attn_path == 2;
  return max_keys <= 512 && (int64_t)nq * max_keys <= 4096;
}

static size_t attn_ws(int nq, int H, int d_v, int entries, int W) {
  if (nq < 1 || H < 1 || d_v < 1) return 0;
  return use_g16(nq, entries + W) ? g16::ws_bytes(nq, H, d_v, entries + W) : plan_attn(nq, H, d_v, entries, W).ws;
}

// Scratch of hybrid_attn_decode_noalloc, defined below.
static int scratch_address(const char* name, void** out);

// Runs one call on the kernel its shape selects. noalloc: the split partials go to the static
// scratch (refused if they need more), ws is ignored.
static int run_attn(const char* name, const AttnCall& c, bool noalloc, void* ws, size_t ws_bytes, hipStream_t s) {
  const int entries = c.N_cap > 0 ? (c.topk ? c.k : c.N_cap) : 0;
  const bool g = use_g16(c.nq, entries + c.W);
  AttnPlan p{};
  if (!g) p = plan_attn(c.nq, c.H, c.d_v, entries, c.W);
  const size_t need = g ? g16::ws_bytes(c.nq, c.H, c.d_v, entries + c.W) : p.ws;
  if (noalloc) {
    CSKV_REQUIRE(need <= (size_t)CSKV_NOALLOC_SCRATCH_BYTES, CSKV_EWORKSPACE,
                 "%s: the key splits need %zu bytes of scratch > the static %zu bytes (use hybrid_attn_decode)",
                 name, need, (size_t)CSKV_NOALLOC_SCRATCH_BYTES);
    ws = nullptr;
    ws_bytes = (size_t)CSKV_NOALLOC_SCRATCH_BYTES;
    if (need > 0) {
      const int rc = scratch_address(name, &ws);
      if (rc) return rc;
    }
  }
  if (g) return g16::launch(name, c, ws, ws_bytes, s);
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
  a.rope_step = pow((double)c.rope_base, -2.0 / (double)c.d_rope);
  a.scale_log2 = c.scale_log2;
  a.q_rms_eps = c.q_rms_eps;
  a.out = c.out;
  a.out_lse = c.out_lse;
  return launch_attn(name, a, p, c.qk_fp4, ws, ws_bytes, s);
}

// Checks the decode arguments and fills the call.
static int decode_setup(const char* name, const uint16_t* q, const int64_t* q_pos, const void* ckv,
                        const void* ckv_scale, int ckv_dtype, int N_cap, const int32_t* n_entries,
                        const int32_t* topk_idx, int k, const uint16_t* win, int W, int B, int H, int D, int d_rope,
                        int d_v, float rope_base, float softmax_scale, uint16_t* out, float* out_lse,
                        float q_rms_eps, int T, int R, AttnCall& c) {
  CSKV_REQUIRE(B >= 1 && N_cap >= 0, CSKV_EINVAL, "%s: B=%d N_cap=%d", name, B, N_cap);
  if (R == 0) R = W;
  CSKV_REQUIRE(T >= 1 && (int64_t)B * T < (1 << 20), CSKV_EINVAL, "%s: T=%d", name, T);
  CSKV_REQUIRE(W == 0 || (int64_t)R >= (int64_t)W + T - 1, CSKV_EINVAL,
               "%s: ring of %d slots < window %d + draft %d - 1", name, R, W, T);
  int rc = check_common(name, H, D, d_rope, d_v, W, ckv_dtype, q_rms_eps);
  if (rc) return rc;
  CSKV_REQUIRE(!topk_idx || k >= 1, CSKV_EINVAL, "%s: k=%d", name, k);
  CSKV_REQUIRE(q && q_pos && out && n_entries, CSKV_EINVAL, "%s: null pointer", name);
  CSKV_REQUIRE(W == 0 || win, CSKV_EINVAL, "%s: null window", name);
  const int kv = ckv_dtype & ~CSKV_QK_FP4;
  CSKV_REQUIRE(N_cap == 0 || (ckv && (kv == CSKV_BF16 || ckv_scale)), CSKV_EINVAL, "%s: null cache", name);
  CSKV_REQUIRE(aligned16(q) && aligned16(ckv) && aligned16(win), CSKV_EINVAL, "%s: q/ckv/win must be 16-byte aligned",
               name);
  c = AttnCall{};
  c.q = q;
  c.q_pos = q_pos;
  c.pos0 = 0;
  c.ckv = ckv;
  c.ckv_scale = ckv_scale;
  c.kv_dtype = kv == CSKV_FP8_E4M3 ? kKvFp8 : (kv == CSKV_MXFP4 ? kKvMxfp4 : kKvBf16);
  c.qk_fp4 = (ckv_dtype & CSKV_QK_FP4) != 0;
  c.N_cap = N_cap;
  c.ckv_seq = N_cap;
  c.n_entries = n_entries;
  c.m = 1;
  c.topk = topk_idx;
  c.k = k;
  c.win = win;
  c.ring = 1;
  c.ring_cap = R;
  c.q_per_seq = T;
  c.W = W;
  c.nq = B * T;
  c.H = H;
  c.D = D;
  c.d_rope = d_rope;
  c.d_v = d_v;
  c.rope_base = rope_base;
  c.scale_log2 = softmax_scale * kLog2e;
  c.q_rms_eps = q_rms_eps;
  c.out = out;
  c.out_lse = out_lse;
  return CSKV_OK;
}

}  // namespace cskv

using namespace cskv;

extern "C" CSKV_API int cskv_attn_path(int path) {
  CSKV_REQUIRE(path >= 0 && path <= 2, CSKV_EINVAL, "cskv_attn_path: path=%d outside [0, 2]", path);
  g_attn_path = path;
  return CSKV_OK;
}

extern "C" CSKV_API int cskv_attn_cu_budget(int cus) {
  CSKV_REQUIRE(cus >= 0 && cus <= 4096, CSKV_EINVAL, "cskv_attn_cu_budget: cus=%d outside [0, 4096]", cus);
  g_attn_cus = cus ? cus : kCUs;
  return CSKV_OK;
}

extern "C" CSKV_API size_t hybrid_attn_decode_workspace_size(int B, int H, int d_v, int N_cap, int k, int W, int dense) {
  if (B < 1 || H < 1 || d_v < 1) return 0;
  return attn_ws(B, H, d_v, N_cap > 0 ? (dense ? N_cap : k) : 0, W);
}

extern "C" CSKV_API int hybrid_attn_decode(const uint16_t* q, const int64_t* q_pos, const void* ckv,
                                           const void* ckv_scale, int ckv_dtype, int N_cap,
                                           const int32_t* n_entries, const int32_t* topk_idx, int k,
                                           const uint16_t* win, int W, int B, int H, int D, int d_rope, int d_v,
                                           float rope_base, float softmax_scale, uint16_t* out, float* out_lse,
                                           void* ws, size_t ws_bytes, float q_rms_eps, int T, int R,
                                           void* stream) {
  const char* name = "hybrid_attn_decode";
  AttnCall c;
  const int rc = decode_setup(name, q, q_pos, ckv, ckv_scale, ckv_dtype, N_cap, n_entries, topk_idx, k, win, W, B, H,
                              D, d_rope, d_v, rope_base, softmax_scale, out, out_lse, q_rms_eps, T, R, c);
  if (rc) return rc;
  return run_attn(name, c, false, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

extern "C" CSKV_API int hybrid_attn_decode_append(const uint16_t* q, const int64_t* q_pos, const void* ckv,
                                                  const void* ckv_scale, int ckv_dtype, int N_cap,
                                                  const int32_t* n_entries, const int32_t* topk_idx, int k,
                                                  uint16_t* ring_x, float* ring_z, const uint16_t* x_new,
                                                  const float* z_new, int W, int B, int H, int D, int d_rope,
                                                  int d_v, float rope_base, float softmax_scale, uint16_t* out,
                                                  float* out_lse, void* ws, size_t ws_bytes, float q_rms_eps, int T,
                                                  int R, void* stream) {
  const char* name = "hybrid_attn_decode_append";
  if (R == 0) R = W;
  CSKV_REQUIRE(ring_x && x_new, CSKV_EINVAL, "%s: null ring or new tokens", name);
  CSKV_REQUIRE(!z_new || ring_z, CSKV_EINVAL, "%s: z_new needs ring_z", name);
  CSKV_REQUIRE(R >= 1 && R >= T, CSKV_EINVAL, "%s: ring of %d slots for %d new tokens", name, R, T);
  CSKV_REQUIRE(B >= 1 && (int64_t)B * R < kNewRow, CSKV_EINVAL, "%s: B=%d rings of %d slots", name, B, R);
  CSKV_REQUIRE(aligned16(x_new), CSKV_EINVAL, "%s: x_new must be 16-byte aligned", name);
  AttnCall c;
  const int rc = decode_setup(name, q, q_pos, ckv, ckv_scale, ckv_dtype, N_cap, n_entries, topk_idx, k, ring_x, W, B,
                              H, D, d_rope, d_v, rope_base, softmax_scale, out, out_lse, q_rms_eps, T, R, c);
  if (rc) return rc;
  c.x_new = x_new;
  c.z_new = z_new;
  c.ring_z = ring_z;
  return run_attn(name, c, false, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

// Scratch of hybrid_attn_decode_noalloc: the key-split partials, in a device array of fixed size.
// Each GPU holds its own copy for the life of the process; its address on a device is looked up
// once, with that device current, and that address (not the host-side name of the array) is what
// the kernels receive.
static __device__ __align__(256) unsigned char scratch[CSKV_NOALLOC_SCRATCH_BYTES];

namespace cskv {

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int scratch_address(const char* name, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  CSKV_REQUIRE(e == hipSuccess, CSKV_EHIP, "%s: hipGetDevice: %s", name, hipGetErrorString(e));
  CSKV_REQUIRE(dev >= 0 && dev < kMaxDevices, CSKV_ENOTSUP, "%s: device %d >= %d", name, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    CSKV_REQUIRE(e == hipSuccess && ptr, CSKV_EHIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", name, dev,
                 hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CSKV_OK;
}

}  // namespace cskv

extern "C" CSKV_API int hybrid_attn_decode_noalloc(const uint16_t* q, const int64_t* q_pos, const void* ckv,
                                                   const void* ckv_scale, int ckv_dtype, int N_cap,
                                                   const int32_t* n_entries, const int32_t* topk_idx, int k,
                                                   const uint16_t* win, int W, int B, int H, int D, int d_rope,
                                                   int d_v, float rope_base, float softmax_scale, uint16_t* out,
                                                   float* out_lse, float q_rms_eps, int T, int R, void* stream) {
  const char* name = "hybrid_attn_decode_noalloc";
  AttnCall c;
  const int rc = decode_setup(name, q, q_pos, ckv, ckv_scale, ckv_dtype, N_cap, n_entries, topk_idx, k, win, W, B, H,
                              D, d_rope, d_v, rope_base, softmax_scale, out, out_lse, q_rms_eps, T, R, c);
  if (rc) return rc;
  return run_attn(name, c, true, nullptr, 0, reinterpret_cast<hipStream_t>(stream));
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
  const int kv = ckv_dtype & ~CSKV_QK_FP4;
  CSKV_REQUIRE(N == 0 || (ckv && (kv == CSKV_BF16 || ckv_scale)), CSKV_EINVAL, "%s: null cache", name);
  CSKV_REQUIRE(aligned16(q) && aligned16(ckv) && aligned16(x), CSKV_EINVAL, "%s: q/ckv/x must be 16-byte aligned",
               name);
  AttnCall c{};
  c.q = q;
  c.q_pos = nullptr;
  c.pos0 = pos0;
  c.ckv = ckv;
  c.ckv_scale = ckv_scale;
  c.kv_dtype = kv == CSKV_FP8_E4M3 ? kKvFp8 : (kv == CSKV_MXFP4 ? kKvMxfp4 : kKvBf16);
  c.qk_fp4 = (ckv_dtype & CSKV_QK_FP4) != 0;
  c.N_cap = N;
  c.ckv_seq = 0;
  c.n_entries = nullptr;
  c.m = m;
  c.topk = topk_idx;
  c.k = k;
  c.win = x;
  c.ring = 0;
  c.ring_cap = W;
  c.q_per_seq = 1;
  c.W = W;
  c.nq = T;
  c.H = H;
  c.D = D;
  c.d_rope = d_rope;
  c.d_v = d_v;
  c.rope_base = rope_base;
  c.scale_log2 = softmax_scale * kLog2e;
  c.q_rms_eps = q_rms_eps;
  c.out = out;
  c.out_lse = out_lse;
  return run_attn(name, c, false, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}
