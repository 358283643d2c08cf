// Lightning indexer (MXFP4 scores on the scaled FP4 MFMA) and exact top-k.
//
// Method: page "DeepSeek-V4가 이차적 어텐션 비용 없이 백만 토큰 컨텍스트를 달성하는
// 방법", section "두 가지 압축 전략: CSA 및 HCA": a light indexer running in FP4
// scores the compressed entries against the query and keeps the top-k (about
// 128) for attention. Score form (DSA lightning indexer):
//   s(t, j) = sum_h w[t,h] * ReLU(q[t,h] . k[j]).
//
// Design. A query's H_I (<= 16) heads form the 16 rows of the A operand of
// v_mfma_scale_f32_16x16x128_f8f6f4 (e2m1 x e2m1, one E8M0 scale per lane =
// per row and 32-wide k block); 16 compressed entries form the columns. Lane l
// loads the 16 contiguous bytes of entry l%16, k-block l/16, so one wave load
// covers 16 whole 64-byte keys (1 KiB contiguous). Products of e2m1 values
// with power-of-two scales are exact and the accumulation stays exact in fp32
// within the documented scale span, so the scores and therefore the top-k are
// exact. ReLU and the head sum run on the accumulator lanes and two xor
// shuffles.
//
// Decode (few queries, long key streams): stage 1 gives each (query, chunk of
// entries) one workgroup that scores the chunk into LDS and keeps the chunk's
// exact top-k; stage 2 merges the chunk winners of each query and writes the
// ordered list. Exactness of the two-stage scheme: an entry of the global top-k
// is beaten by fewer than k keys overall, hence by fewer than k keys of its
// own chunk, so it survives its chunk.
#include "common.cuh"
#include "host_util.h"
#include "topk_select.cuh"

namespace cskv {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kIdxNT = 256;          // threads per workgroup
constexpr int kSub = 4096;           // entries scored per LDS pass
constexpr int kMaxMergeKeys = 8192;  // chunk winners merged per query in stage 2

// max(x, 0) as an integer max on the bit pattern (a negative float, -0 included, has a negative
// pattern): one instruction, no canonicalisation; scores are finite.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// x plus the x of the lane 16 (32) apart, on the VALU: a permlane swap of two copies of x
// exchanges the halves of every 32-lane (64-lane) group, and the two results sum to
// x[l] + x[l ^ 16] (x[l] + x[l ^ 32]) in every lane; no LDS round trip as for a shuffle.
__device__ __forceinline__ float add_xor16(float x) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

__device__ __forceinline__ f32x4 mfma_fp4_acc(uint4 a, uint4 b, int sa, int sb, f32x4 acc) {
  i32x8 va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  i32x8 vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, acc, 4, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ f32x4 mfma_fp4(uint4 a, uint4 b, int sa, int sb) {
  i32x8 va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  i32x8 vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // cbsz = blgp = 4: both operands e2m1
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, acc, 4, 4, 0, sa, 0, sb);
}

struct IndexArgs {
  const uint8_t* iq;
  const uint8_t* iq_scale;
  const float* head_w;
  const uint8_t* ik;
  const uint8_t* ik_scale;
  const int32_t* n_valid;
  int B, T, N_cap, H_I, D_I, k;
  int chunk;     // entries per chunk (multiple of 16)
  int n_chunks;
  uint64_t* part;  // [B*T, n_chunks, k] chunk winners
  int32_t* out_idx;
  float* out_score;
};

template <int CAP>
struct Stage1Smem {
  uint64_t keys[1024 + kSub];
  uint64_t buf[CAP];
  SelectScratch sc;
  __align__(16) uint8_t wsc[kIdxNT / kWave][1024];
};

// Score entries [e_begin, e_end) of one query into keys[0..e_end-e_begin), 16 per wave step.
// KS = number of 128-wide k steps (D_I <= 128 * KS); U = 16-entry groups per wave batch.
// A batch's E8M0 scales (16 * U * D_I/32 bytes <= 1 KiB) arrive with one 16-byte load per
// lane into the wave's LDS slot `wsc` and are read back per group.
template <int KS, int NT, typename Sink, int UU = 0>
__device__ __forceinline__ void score_range_to(const IndexArgs& a, int b, int e_begin, int e_end,
                                               const uint4* qa, const int* qs, const float* hw,
                                               uint8_t* wsc, Sink sink) {
  constexpr int U = UU ? UU : (KS == 1 ? 16 : (KS == 2 ? 8 : 4));
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop control
  const int kb = lane >> 4, col = lane & 15;
  const int kbytes = a.D_I >> 1, sbytes = a.D_I >> 5;
  const uint8_t* ikb = a.ik + (int64_t)b * a.N_cap * kbytes;
  const uint8_t* iksb = a.ik_scale + (int64_t)b * a.N_cap * sbytes;
  const int64_t s_end = (int64_t)a.N_cap * sbytes;  // scale bytes of this sequence
  const int n = e_end - e_begin;
  const int groups = (n + 15) >> 4;
  const int rb = 16 * U * sbytes;                   // scale bytes per batch
  for (int g0 = wave * U; g0 < groups; g0 += (NT / kWave) * U) {
    // scales of entries e_begin + 16*g0 ... (16*U entries)
    {
      const int64_t off = (int64_t)(e_begin + 16 * g0) * sbytes + 16 * lane;
      if (16 * lane < rb) {
        uint4 v = make_uint4(0x7f7f7f7f, 0x7f7f7f7f, 0x7f7f7f7f, 0x7f7f7f7f);
        if (off + 16 <= s_end && ((reinterpret_cast<uintptr_t>(iksb + off) & 15) == 0)) {
          v = *reinterpret_cast<const uint4*>(iksb + off);
        } else {
          uint8_t t[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) t[i] = off + i < s_end ? iksb[off + i] : 127;
          v = *reinterpret_cast<const uint4*>(t);
        }
        *reinterpret_cast<uint4*>(wsc + 16 * lane) = v;
      }
    }
    uint4 kv[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e_begin + (g0 + u) * 16 + col;
      const bool ok = (g0 + u) < groups && e < e_end;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kv[u][s] = make_uint4(0, 0, 0, 0);
        if (ok && (s * 128 + kb * 32) < a.D_I)
          kv[u][s] = ld_stream16(ikb + (int64_t)e * kbytes + s * 64 + kb * 16);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the scale slot is written (wave-local)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u >= groups) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int sc = (s * 128 + kb * 32) < a.D_I ? wsc[(u * 16 + col) * sbytes + s * 4 + kb] : 127;
        acc = mfma_fp4_acc(qa[s], kv[u][s], qs[s], sc, acc);
      }
      // rows 4*kb + r are heads; ReLU, head weight, then sum over the 4 lane groups
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) part = fmaf(hw[r], relu_bits(acc[r]), part);
      part = add_xor32(add_xor16(part));
      const int el = (g0 + u) * 16 + col;
      sink(kb == 0 && el < n, el, make_key(part, (uint32_t)(e_begin + el)));
    }
    __builtin_amdgcn_wave_barrier();  // slot reads done before the next batch overwrites it
  }
}

// Streaming form of the scoring loop (decode kernel A): each wave owns groups of 16 entries
// in batches of U groups and keeps two batches in flight (the next batch is requested before
// the current one is scored). Every load is unconditional, from a clamped address (rows past
// the range repeat its last row and are masked), so that the loads issue back to back and the
// loop carries no branch. A lane's E8M0 scale byte comes from the aligned dword holding it
// (the scale array is 4-byte aligned, so that dword lies inside the array's last dword at most).
template <int KS, int U>
struct KBatch {
  uint4 kv[U][KS];
  uint32_t sc[U][KS];
};

template <int KS, int U>
__device__ __forceinline__ void kbatch_load(const uint8_t* ikb, const uint32_t* sc32, int64_t sc_off0, int kbytes,
                                            int sbytes, int D_I, int e_begin, int e_end, int g, KBatch<KS, U>& B) {
  const int lane = threadIdx.x & (kWave - 1);
  const int kb = lane >> 4, col = lane & 15;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = min(e_begin + (g + u) * 16 + col, e_end - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bool okk = (s * 128 + kb * 32) < D_I;
      B.kv[u][s] = ld_stream16(ikb + (int64_t)e * kbytes + (okk ? s * 64 + kb * 16 : 0));
      B.sc[u][s] = sc32[(sc_off0 + (int64_t)e * sbytes + (okk ? s * 4 + kb : 0)) >> 2];  // dword holding the byte
    }
  }
}

template <int KS, int U, typename Sink>
__device__ __forceinline__ void kbatch_score(const KBatch<KS, U>& B, int64_t sc_off0, int sbytes, int D_I, int e_begin,
                                             int e_end, int groups, int g, const uint4* qa, const int* qs,
                                             const float* hw, Sink& sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int kb = lane >> 4, col = lane & 15;
  const int n = e_end - e_begin;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (g + u >= groups) break;
    const int e = min(e_begin + (g + u) * 16 + col, e_end - 1);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bool okk = (s * 128 + kb * 32) < D_I;
      // lanes past D_I multiply by the zero query operand, so their (real, finite) codes need
      // no masking; only the scale is replaced (an E8M0 byte of 255 would be NaN)
      const int sh = 8 * (int)((sc_off0 + (int64_t)e * sbytes + s * 4 + kb) & 3);
      const int byte = (int)((B.sc[u][s] >> sh) & 255u);
      acc = mfma_fp4_acc(qa[s], B.kv[u][s], qs[s], okk ? byte : 127, acc);
    }
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) part = fmaf(hw[r], relu_bits(acc[r]), part);
    part = add_xor32(add_xor16(part));
    const int el = (g + u) * 16 + col;
    sink(kb == 0 && el < n, el, make_key(part, (uint32_t)(e_begin + el)));
  }
}

template <int KS, int NT, typename Sink>
__device__ __forceinline__ void stream_range_to(const IndexArgs& a, int b, int e_begin, int e_end, const uint4* qa,
                                                const int* qs, const float* hw, Sink sink) {
  // batch size: 8 groups for one 128-wide step (6 in 1024-thread workgroups, whose waves have
  // 128 registers), fewer for wider keys
  constexpr int U = KS == 1 ? (NT > 512 ? 6 : 8) : (KS == 2 ? 2 : 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kbytes = a.D_I >> 1, sbytes = a.D_I >> 5;
  const uint8_t* ikb = a.ik + (int64_t)b * a.N_cap * kbytes;
  const uint32_t* sc32 = reinterpret_cast<const uint32_t*>(a.ik_scale);  // 4-byte aligned
  const int64_t sc_off0 = (int64_t)b * a.N_cap * sbytes;                // this sequence's first scale byte
  const int groups = (e_end - e_begin + 15) >> 4;
  const int stride = (NT / kWave) * U;
  // NB batches per outer step, fully unrolled: batch i+1 is requested before batch i is
  // scored, and no batch is carried across the loop's back edge (which would force the
  // compiler to wait for it there)
  constexpr int NB = 6;
  for (int g0 = wave * U; g0 < groups; g0 += stride * NB) {
    KBatch<KS, U> X[NB];
    kbatch_load<KS, U>(ikb, sc32, sc_off0, kbytes, sbytes, a.D_I, e_begin, e_end, g0, X[0]);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int gi = g0 + i * stride;
      if (gi >= groups) break;
      if (i + 1 < NB) kbatch_load<KS, U>(ikb, sc32, sc_off0, kbytes, sbytes, a.D_I, e_begin, e_end, gi + stride, X[i + 1]);
      kbatch_score<KS, U>(X[i], sc_off0, sbytes, a.D_I, e_begin, e_end, groups, gi, qa, qs, hw, sink);
    }
  }
}

// Keys of [e_begin, e_end) into keys[0..e_end-e_begin).
template <int KS, int NT = kIdxNT, int UU = 0>
__device__ __forceinline__ void score_range(const IndexArgs& a, int b, int e_begin, int e_end,
                                            const uint4* qa, const int* qs, const float* hw,
                                            uint64_t* keys, uint8_t* wsc) {
  auto sink = [keys](bool p, int el, uint64_t key) {
    if (p) keys[el] = key;
  };
  score_range_to<KS, NT, decltype(sink), UU>(a, b, e_begin, e_end, qa, qs, hw, wsc, sink);
}

// Per-lane A operand (query rows) and head weights for query bq.
template <int KS>
__device__ __forceinline__ void load_query(const IndexArgs& a, int bq, uint4* qa, int* qs, float* hw) {
  const int lane = threadIdx.x & (kWave - 1);
  const int kb = lane >> 4, row = lane & 15;
  const int kbytes = a.D_I >> 1, sbytes = a.D_I >> 5;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qa[s] = make_uint4(0, 0, 0, 0);
    qs[s] = 127;
    if (row < a.H_I && (s * 128 + kb * 32) < a.D_I) {
      const int64_t qrow = (int64_t)bq * a.H_I + row;
      qa[s] = *reinterpret_cast<const uint4*>(a.iq + qrow * kbytes + s * 64 + kb * 16);
      qs[s] = a.iq_scale[qrow * sbytes + s * 4 + kb];
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * kb + r;
    hw[r] = h < a.H_I ? (a.head_w ? a.head_w[(int64_t)bq * a.H_I + h] : 1.0f) : 0.0f;
  }
}

// Stage 1: grid (B*T, n_chunks). Chunk winners (exactly k slots, 0-padded) to part.
template <int CAP, int KS>
__global__ __launch_bounds__(kIdxNT) void index_chunk_kernel(IndexArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Stage1Smem<CAP>& sm = *reinterpret_cast<Stage1Smem<CAP>*>(smem_raw);
  const int bq = blockIdx.x;
  const int b = bq / a.T;
  const int chunk = blockIdx.y;
  const int nv = min(a.n_valid[bq], a.N_cap);
  const int c_begin = chunk * a.chunk;
  const int c_end = min(c_begin + a.chunk, nv);
  uint64_t* out = a.part + ((int64_t)bq * a.n_chunks + chunk) * a.k;
  if (c_begin >= c_end) {
    for (int i = threadIdx.x; i < a.k; i += kIdxNT) out[i] = 0;
    return;
  }
  uint4 qa[KS];
  int qs[KS];
  float hw[4];
  load_query<KS>(a, bq, qa, qs, hw);
  int kept = 0;  // running winners in keys[0..kept)
  for (int s0 = c_begin; s0 < c_end; s0 += kSub) {
    const int s1 = min(s0 + kSub, c_end);
    score_range<KS>(a, b, s0, s1, qa, qs, hw, sm.keys + kept, sm.wsc[threadIdx.x >> 6]);
    __syncthreads();
    const int n = kept + (s1 - s0);
    const int kk = min(a.k, n);
    select_topk<kIdxNT, CAP>(sm.keys, n, kk, sm.buf, &sm.sc);
    for (int i = threadIdx.x; i < kk; i += kIdxNT) sm.keys[i] = sm.buf[i];
    __syncthreads();
    kept = kk;
  }
  for (int i = threadIdx.x; i < a.k; i += kIdxNT) out[i] = i < kept ? sm.keys[i] : 0;
}

template <int CAP>
struct Stage2Smem {
  uint64_t keys[kMaxMergeKeys];
  uint64_t buf[CAP];
  SelectScratch sc;
};

// Stage 2: one workgroup per query merges its chunk winners and writes the ordered list.
template <int CAP>
__global__ __launch_bounds__(kIdxNT) void index_merge_kernel(IndexArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Stage2Smem<CAP>& sm = *reinterpret_cast<Stage2Smem<CAP>*>(smem_raw);
  const int bq = blockIdx.x;
  const int nv = min(a.n_valid[bq], a.N_cap);
  const int kk = min(a.k, nv);
  int32_t* oi = a.out_idx + (int64_t)bq * a.k;
  float* os = a.out_score ? a.out_score + (int64_t)bq * a.k : nullptr;
  if (kk > 0) {
    const int n = a.n_chunks * a.k;
    const uint64_t* src = a.part + (int64_t)bq * n;
    for (int i = threadIdx.x; i < n; i += kIdxNT) sm.keys[i] = src[i];
    __syncthreads();
    select_topk<kIdxNT, CAP>(sm.keys, n, kk, sm.buf, &sm.sc);
  }
  for (int i = threadIdx.x; i < a.k; i += kIdxNT) {
    if (i < kk) {
      const uint64_t key = sm.buf[i];
      oi[i] = (int32_t)(~(uint32_t)key);
      if (os) os[i] = ordered_to_score((uint32_t)(key >> 32));
    } else {
      oi[i] = -1;
      if (os) os[i] = -INFINITY;
    }
  }
}

// ---------------------------------------------------------------- decode path (few queries)
//
// Kernel A (grid Q x C, 1024 threads, one workgroup per CU): streams chunk c of query q with
// every wave keeping two batches of loads in flight, keeps all of the chunk's keys in LDS,
// and writes the chunk's top keys to its 2k candidate slots (0 = empty): every key at or
// above the floor of a histogram bin chosen so that at least min(k, chunk) and at most 2k
// keys pass (radix-style refinement over [chunk min, chunk max], 11 bits per level). Kernel B
// (one workgroup per query) runs the same selection over the C * 2k slots down to at most
// kSelCap keys and ranks them. Exactness: an entry of the global top-k is beaten by fewer than
// k keys overall, hence by fewer than k keys of its own chunk, so it is among its chunk's
// passing keys; the top-k of the union of those is the global top-k. No step depends on the
// data's distribution, and nothing is carried between calls.
constexpr int kDecNT = 1024;     // threads of kernel A
constexpr int kFinNT = 512;      // threads of kernel B (fewer waves per barrier)
constexpr int kDecSub = 8448;    // entries a chunk workgroup holds in LDS at once
constexpr int kSelBins = 2048;   // histogram bins per refinement level
constexpr int kSelCap = 1024;    // kernel B: keys ranked directly
constexpr int kStageMax = 8192;  // kernel B: candidate slots staged in LDS
constexpr int kMaxSlots = 2048;  // 2k for k <= 1024

struct DecodeArgs {
  IndexArgs a;
  uint64_t* cand;  // [Q][C][slots] candidate keys, 0 = empty
  int chunk, n_chunks, slots;
};

// Cross-lane integer scans and reductions on DPP row operations (rows of 16 lanes) and
// readlane of the row results, instead of permutes through LDS. Every lane of the wave must be
// active.
template <int CTRL>
__device__ __forceinline__ int dpp_shr0(int x) {  // row shift: lanes shifted in from outside the row read 0
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ int dpp_perm(int x) {  // quad permutation or row rotation (all sources valid)
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}

// Inclusive prefix sum over the lanes of the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_shr0<0x111>(v);  // row_shr:1
  v += dpp_shr0<0x112>(v);  // row_shr:2
  v += dpp_shr0<0x114>(v);  // row_shr:4
  v += dpp_shr0<0x118>(v);  // row_shr:8
  const int r = (threadIdx.x & (kWave - 1)) >> 4;
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31),
            t2 = __builtin_amdgcn_readlane(v, 47);
  return v + (r > 0 ? t0 : 0) + (r > 1 ? t1 : 0) + (r > 2 ? t2 : 0);
}

// Reduction over the lanes of the wave (every lane gets the result).
template <typename Op>
__device__ __forceinline__ int wave_reduce_i32(int v, Op op) {
  v = op(v, dpp_perm<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_perm<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_perm<0x124>(v));  // row_ror:4
  v = op(v, dpp_perm<0x128>(v));  // row_ror:8
  return op(op(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
            op(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  return wave_reduce_i32(v, [](int a, int b) { return a + b; });
}

// Highest bin b (scanning from the top) whose cumulative count reaches kk; returns b and the
// count strictly above it in *above. NT is the block size (<= 1024); NB is a power of two.
// kk >= 1 and total >= kk. scratch holds at least 34 ints. Every thread must call it, after a
// barrier that follows every earlier read of scratch; it ends with a barrier.
template <int NB, int NT>
__device__ int find_threshold_bin(const uint32_t* hist, int kk, int* above, int* scratch) {
  constexpr int PER = NB >= NT ? NB / NT : 1;
  constexpr int ACTIVE = NB / PER;  // threads owning bins
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t >> 6;
  // thread t < ACTIVE owns bins [NB - PER*(t+1), NB - PER*t), the t-th slice from the top
  const int top = NB - PER * t;
  int s = 0;
  if (t < ACTIVE) {
#pragma unroll
    for (int i = 1; i <= PER; ++i) s += hist[top - i];
  }
  const int inc = wave_incl_scan(s);
  if (lane == kWave - 1) scratch[w] = inc;
  if (t == 0) {  // defaults (bin 0) in case the counts do not reach kk
    scratch[32] = 0;
    scratch[33] = 0;
  }
  __syncthreads();
  int wbase = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) wbase += i < w ? scratch[i] : 0;
  const int incl = inc + wbase, excl = incl - s;
  if (t < ACTIVE && excl < kk && incl >= kk) {
    int c = excl;
    for (int i = 1; i <= PER; ++i) {
      const int h = hist[top - i];
      if (c + h >= kk) {
        scratch[32] = top - i;
        scratch[33] = c;
        break;
      }
      c += h;
    }
  }
  __syncthreads();
  *above = scratch[33];
  return scratch[32];
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

struct SelShared {
  uint32_t hist[kSelBins];
  int scratch[34];
  unsigned long long mx, mn;
  int cnt;
  uint32_t mx32, mn32;
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return (uint32_t)wave_reduce_i32((int)v, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return (uint32_t)wave_reduce_i32((int)v, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
}

// Folds per-lane ranges [mn, mx] of ordered scores into ss.mn32 / ss.mx32 (which thread 0 set
// to ~0 / 0 before an earlier barrier). The caller's next barrier publishes them.
__device__ __forceinline__ void fold_score_range(uint32_t mx, uint32_t mn, SelShared& ss) {
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    atomicMax(&ss.mx32, mx);
    atomicMin(&ss.mn32, mn);
  }
}

// Key bounds covering every key whose ordered score lies in [mn32, mx32] (keys are >= 1).
__device__ __forceinline__ void key_bounds(const SelShared& ss, uint64_t* lo, uint64_t* hi) {
  const uint64_t l = (uint64_t)ss.mn32 << 32;
  *lo = l ? l : 1;
  *hi = ((uint64_t)ss.mx32 << 32) | 0xffffffffull;
}

// Register-resident forms: every thread holds PER keys (0 = empty). The floor: at least kk
// nonzero keys at or above it and at most cap (or exactly kk once bins hold single keys).
// hist must be zero on entry; it is zero again on return.
template <int NT, int PER>
__device__ uint64_t reg_select_floor(const uint64_t (&v)[PER], int kk, int cap, uint64_t lo, uint64_t hi,
                                     SelShared& ss) {
  const int tid = threadIdx.x;
  const uint64_t R = hi - lo;
  int shift = R == 0 ? 0 : max(0, 64 - __builtin_clzll(R) - 11);  // (key - lo) >> shift < 2048
  uint64_t base = lo;
  int need = kk, above_all = 0;
  for (;;) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (v[j] >= base) {
        const uint64_t bin = (v[j] - base) >> shift;
        if (bin < (uint64_t)kSelBins) atomicAdd(&ss.hist[bin], 1u);
      }
    }
    __syncthreads();
    int above;
    const int thr = find_threshold_bin<kSelBins, NT>(ss.hist, need, &above, ss.scratch);
    const int in_bin = (int)ss.hist[thr];
    base += (uint64_t)thr << shift;
    above_all += above;
    need -= above;
    __syncthreads();  // histogram reads done before it is cleared
    for (int i = tid; i < kSelBins; i += NT) ss.hist[i] = 0;
    __syncthreads();
    if (above_all + in_bin <= cap || shift == 0) break;
    shift = max(0, shift - 11);
  }
  return base;
}

// Writes the register keys >= base (base >= 1) to dst[0..) (at most cap of them, in no
// particular order) and returns their number. Ends with a barrier.
template <int NT, int PER>
__device__ int reg_compact_ge(const uint64_t (&v)[PER], uint64_t base, uint64_t* dst, int cap, SelShared& ss) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
  int c = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) c += v[j] >= base;
  const int inc = wave_incl_scan(c);
  if (lane == kWave - 1) ss.scratch[w] = inc;
  __syncthreads();
  int off = inc - c, total = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    off += i < w ? ss.scratch[i] : 0;
    total += ss.scratch[i];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (v[j] >= base && off < cap) dst[off++] = v[j];
  __syncthreads();
  return min(total, cap);
}

// Max, min and count of the nonzero keys of keys[0..n) (block-wide, every thread gets them).
template <int NT>
__device__ void block_range(const uint64_t* keys, int n, SelShared& ss, uint64_t* hi, uint64_t* lo, int* cnt) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    ss.mx = 0;
    ss.mn = ~0ull;
    ss.cnt = 0;
  }
  uint64_t mx = 0, mn = ~0ull;
  int c = 0;
  for (int i = tid; i < n; i += NT) {
    const uint64_t v = keys[i];
    if (v) {
      mx = v > mx ? v : mx;
      mn = v < mn ? v : mn;
      ++c;
    }
  }
  mx = wave_max_u64(mx);
  mn = ~wave_max_u64(~mn);
  c = wave_sum_i32(c);
  __syncthreads();
  if ((tid & (kWave - 1)) == 0) {
    atomicMax(&ss.mx, (unsigned long long)mx);
    atomicMin(&ss.mn, (unsigned long long)mn);
    atomicAdd(&ss.cnt, c);
  }
  __syncthreads();
  *hi = ss.mx;
  *lo = ss.mn;
  *cnt = ss.cnt;
}

// Lower edge of a histogram bin such that at least kk of the nonzero keys of keys[0..n) lie at
// or above it and at most cap do (or exactly kk when the last level has single-key bins).
// Requires kk <= (number of nonzero keys) and lo <= every nonzero key <= hi.
template <int NT>
__device__ uint64_t select_floor(const uint64_t* keys, int n, int kk, int cap, uint64_t lo, uint64_t hi,
                                 SelShared& ss) {
  const int tid = threadIdx.x;
  const uint64_t R = hi - lo;
  int shift = R == 0 ? 0 : max(0, 64 - __builtin_clzll(R) - 11);  // (key - lo) >> shift < 2048
  uint64_t base = lo;
  int need = kk, above_all = 0;
  for (;;) {
    for (int i = tid; i < kSelBins; i += NT) ss.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint64_t v = keys[i];
      if (v >= base) {
        const uint64_t bin = (v - base) >> shift;
        if (bin < (uint64_t)kSelBins) atomicAdd(&ss.hist[bin], 1u);
      }
    }
    __syncthreads();
    int above;
    const int thr = find_threshold_bin<kSelBins, NT>(ss.hist, need, &above, ss.scratch);
    const int in_bin = (int)ss.hist[thr];
    base += (uint64_t)thr << shift;
    above_all += above;
    need -= above;
    __syncthreads();  // histogram reads done before it is cleared
    if (above_all + in_bin <= cap || shift == 0) break;
    shift = max(0, shift - 11);
  }
  return base;
}

struct ChunkSmem {
  uint64_t keys[kMaxSlots + kDecSub];  // carried keys + one sub-chunk
  SelShared ss;
};

// Kernel A: grid (Q, C). Candidate slots of chunk c of query q.
template <int KS>
__global__ __launch_bounds__(kDecNT) void index_chunk_decode_kernel(DecodeArgs d) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  ChunkSmem& sm = *reinterpret_cast<ChunkSmem*>(smem_raw);
  constexpr int PER = (kMaxSlots + kDecSub + kDecNT - 1) / kDecNT;
  const IndexArgs& a = d.a;
  const int q = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  const int b = q / a.T;
  const int nv = min(a.n_valid[q], a.N_cap);
  const int kk = min(a.k, nv);
  const int c0 = c * d.chunk, c1 = min(c0 + d.chunk, nv);
  uint64_t* out = d.cand + ((int64_t)q * d.n_chunks + c) * d.slots;
  for (int i = tid; i < kSelBins; i += kDecNT) sm.ss.hist[i] = 0;
  if (tid == 0) {
    sm.ss.mx32 = 0;
    sm.ss.mn32 = ~0u;
  }
  uint4 qa[KS];
  int qs[KS];
  float hw[4];
  load_query<KS>(a, q, qa, qs, hw);
  uint32_t mx = 0, mn = ~0u;  // this lane's range of ordered scores (for the histogram bounds)
  int kept = 0;               // keys in sm.keys[0..kept)
  for (int s0 = c0; s0 < c1; s0 += kDecSub) {
    const int s1 = min(s0 + kDecSub, c1);
    uint64_t* dst = sm.keys + kept;
    stream_range_to<KS, kDecNT>(a, b, s0, s1, qa, qs, hw, [dst, &mx, &mn](bool p, int el, uint64_t key) {
      if (p) {
        dst[el] = key;
        const uint32_t sc = (uint32_t)(key >> 32);
        mx = max(mx, sc);
        mn = min(mn, sc);
      }
    });
    fold_score_range(mx, mn, sm.ss);
    __syncthreads();
    const int n = kept + (s1 - s0);
    kept = n;
    if (n > d.slots) {  // keep the keys at or above a floor that keeps this chunk's top-kk
      uint64_t v[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = tid + j * kDecNT;
        const uint64_t x = sm.keys[min(i, kMaxSlots + kDecSub - 1)];  // unconditional: all reads in flight
        v[j] = i < n ? x : 0;
      }
      uint64_t lo, hi;
      key_bounds(sm.ss, &lo, &hi);
      const uint64_t base = reg_select_floor<kDecNT, PER>(v, kk, d.slots, lo, hi, sm.ss);
      kept = reg_compact_ge<kDecNT, PER>(v, base, sm.keys, d.slots, sm.ss);
    }
  }
  for (int i = tid; i < d.slots; i += kDecNT) out[i] = i < kept ? sm.keys[i] : 0;
}

struct FinalSmem {
  uint64_t keys[kStageMax];
  uint64_t sel[kSelCap];
  int rk[kSelCap];
  SelShared ss;
};

// Ranks sel[0..m) (distinct keys, m <= kSelCap) and writes the ones of rank < kk to their
// slots. Each thread takes two keys and counts the greater keys in a 1/P slice, comparing every
// key it reads with both (P = min(NT, 2 NT / m') threads per key pair, m' = m rounded up to a
// power of two, so the pairs advance by at least one per step); the partial ranks meet in an
// LDS counter.
template <int NT>
__device__ __forceinline__ void rank_write(const uint64_t* sel, int m, int kk, int32_t* oi, float* os, int* rk) {
  constexpr int KPT = 2;
  const int tid = threadIdx.x;
  m = __builtin_amdgcn_readfirstlane(m);
  int mp = 1;
  while (mp < m) mp <<= 1;
  const int P = mp >= NT * KPT ? 1 : min(NT, NT * KPT / mp);  // threads per key pair (power of two, <= NT)
  for (int i = tid; i < m; i += NT) rk[i] = 0;
  __syncthreads();
  const int part = tid % P, slice = (m + P - 1) / P;
  const int j0 = part * slice, j1 = min(m, j0 + slice);
  for (int ib = (tid / P) * KPT; ib < m; ib += (NT / P) * KPT) {
    uint64_t key[KPT];
    int r[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      key[u] = ib + u < m ? sel[ib + u] : ~0ull;  // no key is greater than ~0
      r[u] = 0;
    }
    for (int jx = j0; jx < j1; ++jx) {
      const uint64_t x = sel[jx];
#pragma unroll
      for (int u = 0; u < KPT; ++u) r[u] += x > key[u];
    }
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if (ib + u < m && r[u]) atomicAdd(&rk[ib + u], r[u]);
  }
  __syncthreads();
  for (int i = tid; i < m; i += NT) {
    const int rank = rk[i];
    if (rank < kk) {
      const uint64_t key = sel[i];
      oi[rank] = (int32_t)(~(uint32_t)key);
      if (os) os[rank] = ordered_to_score((uint32_t)(key >> 32));
    }
  }
}

// Kernel B: one workgroup per query; the ordered top-k of its C * slots candidates.
__global__ __launch_bounds__(kFinNT) void index_final_decode_kernel(DecodeArgs d) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FinalSmem& sm = *reinterpret_cast<FinalSmem*>(smem_raw);
  constexpr int PER = kStageMax / kFinNT;
  const IndexArgs& a = d.a;
  const int q = blockIdx.x, tid = threadIdx.x;
  const int nv = min(a.n_valid[q], a.N_cap);
  const int kk = min(a.k, nv);
  int32_t* oi = a.out_idx + (int64_t)q * a.k;
  float* os = a.out_score ? a.out_score + (int64_t)q * a.k : nullptr;
  for (int i = kk + tid; i < a.k; i += kFinNT) {  // padding
    oi[i] = -1;
    if (os) os[i] = -INFINITY;
  }
  if (kk == 0) return;
  const int n = d.n_chunks * d.slots;
  const uint64_t* src = d.cand + (int64_t)q * n;
  if (n <= kStageMax) {
    // register-resident: every slot is loaded once, all loads in flight together
    for (int i = tid; i < kSelBins; i += kFinNT) sm.ss.hist[i] = 0;
    if (tid == 0) {
      sm.ss.mx32 = 0;
      sm.ss.mn32 = ~0u;
      sm.ss.cnt = 0;
    }
    uint64_t v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * kFinNT;
      v[j] = i < n ? src[i] : 0;
    }
    uint32_t mx = 0, mn = ~0u;
    int nz = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (v[j]) {
        const uint32_t sc = (uint32_t)(v[j] >> 32);
        mx = max(mx, sc);
        mn = min(mn, sc);
        ++nz;
      }
    }
    nz = wave_sum_i32(nz);
    __syncthreads();  // range words initialised
    fold_score_range(mx, mn, sm.ss);
    if ((tid & (kWave - 1)) == 0) atomicAdd(&sm.ss.cnt, nz);
    __syncthreads();
    uint64_t lo, hi;
    key_bounds(sm.ss, &lo, &hi);
    const uint64_t base = sm.ss.cnt <= kSelCap ? lo : reg_select_floor<kFinNT, PER>(v, kk, kSelCap, lo, hi, sm.ss);
    const int m = reg_compact_ge<kFinNT, PER>(v, base, sm.sel, kSelCap, sm.ss);
    rank_write<kFinNT>(sm.sel, m, kk, oi, os, sm.rk);
    return;
  }
  // large candidate lists: histogram passes over global memory
  uint64_t hi, lo;
  int nz;
  block_range<kFinNT>(src, n, sm.ss, &hi, &lo, &nz);
  const uint64_t base = nz <= kSelCap ? lo : select_floor<kFinNT>(src, n, kk, kSelCap, lo, hi, sm.ss);
  const int lane = tid & (kWave - 1), w = tid >> 6;
  int cnt = 0;
  for (int i = tid; i < n; i += kFinNT) cnt += src[i] >= base;
  const int inc = wave_incl_scan(cnt);
  if (lane == kWave - 1) sm.ss.scratch[w] = inc;
  __syncthreads();
  int off = inc - cnt, m = 0;
#pragma unroll
  for (int i = 0; i < kFinNT / kWave; ++i) {
    off += i < w ? sm.ss.scratch[i] : 0;
    m += sm.ss.scratch[i];
  }
  m = min(m, kSelCap);
  for (int i = tid; i < n; i += kFinNT) {
    const uint64_t v = src[i];
    if (v >= base && off < kSelCap) sm.sel[off++] = v;
  }
  __syncthreads();
  rank_write<kFinNT>(sm.sel, m, kk, oi, os, sm.rk);
}

// Chunking of kernel A: one workgroup per CU for the whole job (256), chunks of at most
// kDecSub entries (one LDS pass), multiples of 16.
static void decode_chunks(int queries, int N_cap, int* chunk, int* n_chunks) {
  int n = 256 / queries;
  const int by_lds = (N_cap + kDecSub - 1) / kDecSub;
  if (n < by_lds) n = by_lds;
  if (n < 1) n = 1;
  int c = (N_cap + n - 1) / n;
  c = (c + 15) & ~15;
  if (c < 16) c = 16;
  *chunk = c;
  *n_chunks = (N_cap + c - 1) / c;
}

static size_t decode_ws_bytes(int queries, int N_cap, int k) {
  int chunk, n_chunks;
  decode_chunks(queries, N_cap, &chunk, &n_chunks);
  return (size_t)queries * n_chunks * (2 * k) * sizeof(uint64_t);
}

template <int KS>
static void launch_decode_ks(const DecodeArgs& d, int queries, hipStream_t s) {
  const size_t smem_a = sizeof(ChunkSmem), smem_b = sizeof(FinalSmem);
  (void)hipFuncSetAttribute((const void*)index_chunk_decode_kernel<KS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem_a);
  (void)hipFuncSetAttribute((const void*)index_final_decode_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem_b);
  hipLaunchKernelGGL((index_chunk_decode_kernel<KS>), dim3(queries, d.n_chunks), dim3(kDecNT), smem_a, s, d);
  hipLaunchKernelGGL(index_final_decode_kernel, dim3(queries), dim3(kFinNT), smem_b, s, d);
}

static int launch_decode(const IndexArgs& a, int queries, int ks, void* ws, hipStream_t s) {
  DecodeArgs d;
  d.a = a;
  decode_chunks(queries, a.N_cap > 0 ? a.N_cap : 1, &d.chunk, &d.n_chunks);
  d.slots = 2 * a.k;
  d.cand = reinterpret_cast<uint64_t*>(ws);
  if (ks == 1)
    launch_decode_ks<1>(d, queries, s);
  else if (ks == 2)
    launch_decode_ks<2>(d, queries, s);
  else
    launch_decode_ks<4>(d, queries, s);
  CSKV_LAUNCH_CHECK("csa_index_topk (decode)");
  return CSKV_OK;
}

// ---------------------------------------------------------------- decode path, draft queries
//
// A decode step that checks T > 1 draft tokens has T queries per sequence, query t seeing the
// first n_valid[b, t] entries. Kernel M (grid B * ceil(T / TQ) x C, 1024 threads) gives a
// workgroup TQ consecutive queries of one sequence (H_I <= 8: two queries per MFMA row tile,
// TQ / 2 row tiles) and streams chunk c of that sequence's keys once for all of them. Each
// query's scores are kept in LDS by entry position (the entry index is implied by it), then one
// selection pass serves all TQ queries at once: kernel A's histogram levels with one histogram
// per query, scanned by a thread group per query, every barrier shared. The slots each query
// gets for the chunk, and kernel B's merge per query, are kernel A's.
constexpr int kMqSub = 8448;   // entries of one chunk (LDS holds TQ scores of each)
constexpr int kMqBins = 1024;  // histogram bins per level and query (10 bits)
constexpr int kMqU = 6;        // groups of 16 entries per wave and batch

template <int TQ>
struct MqSmem {
  uint32_t sc[TQ][kMqSub];  // ordered scores of the chunk's entries (0: not visible)
  uint32_t hist[TQ][kMqBins];
  int scratch[TQ][kDecNT / kWave];
  int thr[TQ], above[TQ];
  uint32_t mx32[TQ], mn32[TQ];
};

// Bin b of hist[j] (scanning from the top) whose cumulative count reaches need[j], and the count
// strictly above it, for every active query j: thread group j (NT / TQ threads) scans hist[j].
// Every thread calls it after a barrier that follows the histogram's last update and every
// earlier read of the results; it ends with a barrier.
// nj, aj: need and activity of this thread's query (tid / (NT / TQ)).
template <int TQ, int NT>
__device__ void mq_threshold_bins(MqSmem<TQ>& sm, int nj, bool aj) {
  constexpr int GT = NT / TQ;             // threads per query
  constexpr int PB = kMqBins / GT;        // bins per thread
  constexpr int WPG = GT / kWave;         // waves per query
  static_assert(PB >= 1 && WPG >= 1, "group shape");
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
  const int j = tid / GT, lt = tid - j * GT;
  const int top = kMqBins - PB * lt;  // this thread's bins: [top - PB, top)
  if (tid < TQ) {  // defaults (bin 0) in case the counts do not reach need
    sm.thr[tid] = 0;
    sm.above[tid] = 0;
  }
  int sum = 0;
#pragma unroll
  for (int i = 1; i <= PB; ++i) sum += (int)sm.hist[j][top - i];
  const int inc = wave_incl_scan(sum);
  if (lane == kWave - 1) sm.scratch[0][w] = inc;
  __syncthreads();
  int wbase = 0;
  const int w0 = j * WPG;
#pragma unroll
  for (int i = 0; i < WPG; ++i) wbase += w0 + i < w ? sm.scratch[0][w0 + i] : 0;
  const int incl = inc + wbase, excl = incl - sum;
  if (aj && excl < nj && incl >= nj) {
    int c = excl;
    for (int i = 1; i <= PB; ++i) {
      const int h = (int)sm.hist[j][top - i];
      if (c + h >= nj) {
        sm.thr[j] = top - i;
        sm.above[j] = c;
        break;
      }
      c += h;
    }
  }
  __syncthreads();
}

template <int TQ>
__global__ __launch_bounds__(kDecNT) void index_chunk_multi_kernel(DecodeArgs d, int ngroups) {
  constexpr int NRT = TQ / 2;                 // row tiles: two queries (8 rows each) per tile
  constexpr int PER = (kMqSub + kDecNT - 1) / kDecNT;
  constexpr int U = kMqU, NB = 6;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  MqSmem<TQ>& sm = *reinterpret_cast<MqSmem<TQ>*>(smem_raw);
  const IndexArgs& a = d.a;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, col = lane & 15;
  const int b = blockIdx.x / ngroups, t0 = (blockIdx.x - b * ngroups) * TQ, c = blockIdx.y;
  // the group's queries: visible entries and the number kept per chunk
  int nv[TQ], kk[TQ];
#pragma unroll
  for (int j = 0; j < TQ; ++j) {
    const int t = t0 + j;
    nv[j] = t < a.T ? min(a.n_valid[(int64_t)b * a.T + t], a.N_cap) : 0;
    kk[j] = min(a.k, nv[j]);
  }
  int cmax = 0;
#pragma unroll
  for (int j = 0; j < TQ; ++j) cmax = max(cmax, nv[j]);
  const int c0 = c * d.chunk, c1 = min(c0 + d.chunk, cmax);  // entries [c0, c1) seen by someone
  const int n_el = max(0, c1 - c0);
  for (int i = tid; i < TQ * kMqBins; i += kDecNT) (&sm.hist[0][0])[i] = 0;
  if (tid < TQ) {
    sm.mx32[tid] = 0;
    sm.mn32[tid] = ~0u;
  }
  // A operand: row tile rt, lane row col = query 2 rt + col / 8, head col % 8
  uint4 qa[NRT];
  int qs[NRT];
  float hw[NRT][4];
  int nvl[NRT];  // entries visible to the query whose scores this lane writes (G = 0, 2)
  const int kbytes = a.D_I >> 1, sbytes = a.D_I >> 5;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int ta = t0 + 2 * rt + col / 8, ha = col % 8;
    const bool oka = ta < a.T && ha < a.H_I && G * 32 < a.D_I;
    const int64_t qrow = ((int64_t)b * a.T + ta) * a.H_I + ha;
    qa[rt] = oka ? *reinterpret_cast<const uint4*>(a.iq + qrow * kbytes + G * 16) : make_uint4(0, 0, 0, 0);
    qs[rt] = oka ? (int)a.iq_scale[qrow * sbytes + G] : 127;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * G + r, tr = t0 + 2 * rt + row / 8, hr = row % 8;
      hw[rt][r] = (tr < a.T && hr < a.H_I) ? (a.head_w ? a.head_w[((int64_t)b * a.T + tr) * a.H_I + hr] : 1.0f) : 0.0f;
    }
    const int jl = 2 * rt + (G >> 1);
    int v = nv[0];
#pragma unroll
    for (int j = 1; j < TQ; ++j) v = jl == j ? nv[j] : v;
    nvl[rt] = v;
  }

  // stream the chunk once: every wave keeps two batches of loads in flight; each group of 16
  // entries takes NRT MFMAs, and lanes of groups 0 / 2 store the scores of the row tile's two
  // queries
  const uint8_t* ikb = a.ik + (int64_t)b * a.N_cap * kbytes;
  const uint32_t* sc32 = reinterpret_cast<const uint32_t*>(a.ik_scale);
  const int64_t sc_off0 = (int64_t)b * a.N_cap * sbytes;
  const int groups = (n_el + 15) >> 4;
  const int stride = (kDecNT / kWave) * U;
  for (int g0 = wave * U; g0 < groups; g0 += stride * NB) {
    KBatch<1, U> X[NB];
    kbatch_load<1, U>(ikb, sc32, sc_off0, kbytes, sbytes, a.D_I, c0, c1, g0, X[0]);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int gi = g0 + i * stride;
      if (gi >= groups) break;
      if (i + 1 < NB) kbatch_load<1, U>(ikb, sc32, sc_off0, kbytes, sbytes, a.D_I, c0, c1, gi + stride, X[i + 1]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (gi + u >= groups) break;
        const int el = (gi + u) * 16 + col;
        const int e = min(c0 + el, c1 - 1);
        const bool okk = G * 32 < a.D_I;
        const int sh = 8 * (int)((sc_off0 + (int64_t)e * sbytes + G) & 3);
        const int byte = okk ? (int)((X[i].sc[u][0] >> sh) & 255u) : 127;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const f32x4 acc = mfma_fp4(qa[rt], X[i].kv[u][0], qs[rt], byte);
          float part = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) part = fmaf(hw[rt][r], relu_bits(acc[r]), part);
          part = add_xor16(part);
          if ((G & 1) == 0 && el < n_el)
            sm.sc[2 * rt + (G >> 1)][el] = c0 + el < nvl[rt] ? score_to_ordered(part) : 0u;
        }
      }
    }
  }
  __syncthreads();

  // keys in registers (thread tid holds entries tid + i * NT), their score range per query;
  // every read is issued before any is used, and the loop has no branch
  uint64_t v[TQ][PER];
#pragma unroll
  for (int j = 0; j < TQ; ++j) {
    uint32_t o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = sm.sc[j][min(tid + i * kDecNT, kMqSub - 1)];
    uint32_t mx = 0, mn = ~0u;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int el = tid + i * kDecNT;
      const uint32_t x = el < n_el ? o[i] : 0u;
      v[j][i] = x ? (((uint64_t)x << 32) | (uint64_t)(~(uint32_t)(c0 + el))) : 0ull;
      mx = max(mx, x);
      mn = min(mn, x ? x : ~0u);
    }
    mx = wave_max_u32(mx);
    mn = wave_min_u32(mn);
    if (lane == 0) {
      atomicMax(&sm.mx32[j], mx);
      atomicMin(&sm.mn32[j], mn);
    }
  }
  __syncthreads();
  // per query: keys at or above base pass; refine while more than the slots would
  uint64_t base[TQ];
  int shift[TQ], need[TQ], above_all[TQ];
  bool active[TQ];
#pragma unroll
  for (int j = 0; j < TQ; ++j) {
    const uint64_t l = (uint64_t)sm.mn32[j] << 32;
    const uint64_t lo = l ? l : 1, hi = ((uint64_t)sm.mx32[j] << 32) | 0xffffffffull;
    const int n_j = max(0, min(c1, nv[j]) - c0);  // visible entries of the chunk
    base[j] = lo;
    const uint64_t R = hi - lo;
    shift[j] = R == 0 ? 0 : max(0, 64 - __builtin_clzll(R) - 10);
    need[j] = kk[j];
    above_all[j] = 0;
    active[j] = n_j > d.slots && kk[j] > 0;
  }
  // first level on the threads' largest keys only: the kk-th largest of them is at most the
  // kk-th largest key (those kk maxima are kk distinct keys), so the lower edge of its bin is a
  // floor every answer key clears; the levels below then count only the keys above it
  {
    bool any = false;
#pragma unroll
    for (int j = 0; j < TQ; ++j) any = any || active[j];
    if (any) {
#pragma unroll
      for (int j = 0; j < TQ; ++j) {
        if (!active[j]) continue;
        uint64_t tm = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) tm = v[j][i] > tm ? v[j][i] : tm;
        if (tm) atomicAdd(&sm.hist[j][(tm - base[j]) >> shift[j]], 1u);
      }
      __syncthreads();
      {
        const int jt = tid / (kDecNT / TQ);
        int nj = need[0];
        bool aj = active[0];
#pragma unroll
        for (int j = 1; j < TQ; ++j) {
          nj = jt == j ? need[j] : nj;
          aj = jt == j ? active[j] : aj;
        }
        mq_threshold_bins<TQ, kDecNT>(sm, nj, aj);
      }
#pragma unroll
      for (int j = 0; j < TQ; ++j) {
        if (!active[j]) continue;
        base[j] += (uint64_t)sm.thr[j] << shift[j];
        const uint64_t R = (((uint64_t)sm.mx32[j] << 32) | 0xffffffffull) - base[j];
        shift[j] = R == 0 ? 0 : max(0, 64 - __builtin_clzll(R) - 10);
      }
      __syncthreads();  // result reads done before the histogram is cleared
      for (int i = tid; i < TQ * kMqBins; i += kDecNT) (&sm.hist[0][0])[i] = 0;
      __syncthreads();
    }
  }
  for (;;) {
    bool any = false;
#pragma unroll
    for (int j = 0; j < TQ; ++j) any = any || active[j];
    if (!any) break;
#pragma unroll
    for (int j = 0; j < TQ; ++j) {
      if (!active[j]) continue;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (v[j][i] >= base[j]) {
          const uint64_t bin = (v[j][i] - base[j]) >> shift[j];
          if (bin < (uint64_t)kMqBins) atomicAdd(&sm.hist[j][bin], 1u);
        }
      }
    }
    __syncthreads();
    {
      const int jt = tid / (kDecNT / TQ);  // the query whose histogram this thread scans
      int nj = need[0];
      bool aj = active[0];
#pragma unroll
      for (int j = 1; j < TQ; ++j) {
        nj = jt == j ? need[j] : nj;
        aj = jt == j ? active[j] : aj;
      }
      mq_threshold_bins<TQ, kDecNT>(sm, nj, aj);
    }
#pragma unroll
    for (int j = 0; j < TQ; ++j) {
      if (!active[j]) continue;
      const int thr = sm.thr[j], above = sm.above[j];
      const int in_bin = (int)sm.hist[j][thr];
      base[j] += (uint64_t)thr << shift[j];
      above_all[j] += above;
      need[j] -= above;
      if (above_all[j] + in_bin <= d.slots || shift[j] == 0)
        active[j] = false;
      else
        shift[j] = max(0, shift[j] - 10);
    }
    __syncthreads();  // histogram and result reads done before they are cleared
    for (int i = tid; i < TQ * kMqBins; i += kDecNT) (&sm.hist[0][0])[i] = 0;
    __syncthreads();
  }
  // each query's keys at or above its base, to its slots (the rest 0): one scan per query,
  // all behind one barrier
  const int w = tid >> 6;
  int cnt[TQ], inc[TQ];
#pragma unroll
  for (int j = 0; j < TQ; ++j) {
    cnt[j] = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) cnt[j] += v[j][i] >= base[j] && v[j][i] != 0;
    inc[j] = wave_incl_scan(cnt[j]);
    if (lane == kWave - 1) sm.scratch[j][w] = inc[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < TQ; ++j) {
    const int t = t0 + j;
    if (t >= a.T) continue;
    int off = inc[j] - cnt[j], total = 0;
#pragma unroll
    for (int i = 0; i < kDecNT / kWave; ++i) {
      off += i < w ? sm.scratch[j][i] : 0;
      total += sm.scratch[j][i];
    }
    uint64_t* out = d.cand + (((int64_t)b * a.T + t) * d.n_chunks + c) * d.slots;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (v[j][i] >= base[j] && v[j][i] != 0 && off < d.slots) out[off++] = v[j][i];
    for (int i = min(total, d.slots) + tid; i < d.slots; i += kDecNT) out[i] = 0;
  }
}

// Kernel M's chunking: about one workgroup per CU for the whole job, chunks of at most kMqSub
// entries (multiples of 16).
static void multi_chunks(int groups, int N_cap, int* chunk, int* n_chunks) {
  int n = (256 + groups - 1) / groups;
  const int by_lds = (N_cap + kMqSub - 1) / kMqSub;
  if (n < by_lds) n = by_lds;
  if (n < 1) n = 1;
  int c = (N_cap + n - 1) / n;
  c = (c + 15) & ~15;
  if (c < 16) c = 16;
  *chunk = c;
  *n_chunks = (N_cap + c - 1) / c;
}

// Draft steps take kernel M when a row tile holds two queries and a chunk's scores fit LDS.
static bool use_multi(int B, int T, int H_I, int D_I, int k) {
  return T >= 2 && H_I <= 8 && D_I <= 128 && 2 * k <= kMaxSlots / 4 && (int64_t)B * T <= 256;
}
static int multi_tq(int T) { return T <= 2 ? 2 : 4; }

static size_t multi_ws_bytes(int B, int T, int N_cap, int k) {
  const int tq = multi_tq(T), groups = B * ((T + tq - 1) / tq);
  int chunk, n_chunks;
  multi_chunks(groups, N_cap, &chunk, &n_chunks);
  return (size_t)B * T * n_chunks * (2 * k) * sizeof(uint64_t);
}

template <int TQ>
static void launch_multi_tq(const DecodeArgs& d, int B, int ngroups, hipStream_t s) {
  const size_t smem = sizeof(MqSmem<TQ>), smem_b = sizeof(FinalSmem);
  (void)hipFuncSetAttribute((const void*)index_chunk_multi_kernel<TQ>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
  (void)hipFuncSetAttribute((const void*)index_final_decode_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem_b);
  hipLaunchKernelGGL(index_chunk_multi_kernel<TQ>, dim3(B * ngroups, d.n_chunks), dim3(kDecNT), smem, s, d, ngroups);
  hipLaunchKernelGGL(index_final_decode_kernel, dim3(B * d.a.T), dim3(kFinNT), smem_b, s, d);
}

static int launch_multi(const IndexArgs& a, void* ws, hipStream_t s) {
  DecodeArgs d;
  d.a = a;
  const int tq = multi_tq(a.T), ngroups = (a.T + tq - 1) / tq;
  multi_chunks(a.B * ngroups, a.N_cap > 0 ? a.N_cap : 1, &d.chunk, &d.n_chunks);
  d.slots = 2 * a.k;
  d.cand = reinterpret_cast<uint64_t*>(ws);
  if (tq == 2)
    launch_multi_tq<2>(d, a.B, ngroups, s);
  else
    launch_multi_tq<4>(d, a.B, ngroups, s);
  CSKV_LAUNCH_CHECK("csa_index_topk (draft queries)");
  return CSKV_OK;
}

// ---------------------------------------------------------------- many-queries path (prefill)
//
// Kernel P (grid B*ceil(T/QB) x C, 512 threads): a workgroup takes QB consecutive queries of
// one sequence and streams the entries of chunk c that any of them can see through LDS, one
// tile of KT entries at a time, so an entry is read once per QB queries instead of once per
// query. Each wave owns two row tiles of the MFMA; with H_I <= 8 a row tile holds two queries
// (8 rows each), so a wave scores four queries per group of 16 entries. Each query keeps its
// candidates in an LDS buffer: a key joins when it is at or above the query's threshold, a key
// value that at least k keys of the buffer reached when it was last reduced, so the buffer
// always contains the query's top-k of the entries seen so far. A wave reduces a buffer of its
// own queries when the next tile could overflow it, to between k and k + 64 keys (a pivot
// search over the keys with ballot counts; keys are distinct), and at the end ranks the
// survivors and writes the k best (one chunk), or writes them as the chunk's k winners for the
// merge kernel (several chunks; the two-stage exactness argument of the decode path applies).
constexpr int kPfNT = 512;
constexpr int kPfWaves = kPfNT / kWave;
constexpr int kPfRT = 2;          // MFMA row tiles per wave
constexpr int kPfCap = 512;       // candidate slots per query
constexpr int kPfKMax = 128;      // k on this path
constexpr int kPfPL = kPfCap / kWave;
constexpr int kPfU = 8;           // entry groups (of 16) per scoring step
constexpr int kPfHB = 256;        // bins of a wave's threshold histogram
constexpr int kPfMargin = 64;     // a reduction leaves between k and k + kPfMargin keys
constexpr int kPfRankPL = (kPfKMax + kPfMargin + kWave - 1) / kWave;  // survivors ranked per lane
constexpr int kPfTileBytes = 10240;  // key codes of one tile (KT x pitch)

template <int KS>
struct PfTile {
  static constexpr int KT = KS == 1 ? 128 : (KS == 2 ? 64 : 32);  // entries per tile
};
// a buffer is reduced (to k keys) when the next tile could overflow it; between reductions
// at least kPfCap - KT - k keys join, which keeps reductions rare once the threshold settles
static_assert(kPfCap - 128 - kPfKMax - kPfMargin >= 192, "room between reductions");

template <int QB>
struct PfSmem {
  __align__(16) uint8_t kt[2][kPfTileBytes + 256];  // codes, row pitch = kbytes + 16 (+ read slack)
  __align__(16) uint8_t st[2][512];                 // E8M0 scales, KT x sbytes
  uint64_t cand[QB][kPfCap];
  int nv[QB];
  __align__(16) uint32_t hist[kPfWaves][kPfHB];  // one threshold histogram per wave
};

// A threshold th with kk <= #{key >= th} <= kk + margin among the n distinct keys buf[0..n)
// (1 <= kk <= n <= kPfCap), by one wave. Invariant: count(lo) >= kk > count(hi). Each step
// takes as pivot a key strictly inside (lo, hi) (the first such key of the lowest lane that
// holds one; the buffer order is unrelated to the key order) and counts the keys at or above
// it with one comparison, ballot and popcount per slot. While count(lo) > kk + margin >= kk +
// 1 there are at least two keys in [lo, hi), so a pivot exists. The result is at or below the
// kk-th largest key (count >= kk).
__device__ uint64_t wave_threshold(const uint64_t* buf, int n, int kk, int margin) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t v[kPfPL];
#pragma unroll
  for (int i = 0; i < kPfPL; ++i) v[i] = lane + kWave * i < n ? buf[lane + kWave * i] : 0;
  uint64_t lo = 0, hi = ~0ull;  // every key is >= 0; none reaches ~0 (an ordered score never does)
  int clo = n;
  while (clo > kk + margin) {
    uint64_t cand = 0;
    bool found = false;
#pragma unroll
    for (int i = kPfPL - 1; i >= 0; --i) {
      const bool in = lane + kWave * i < n && v[i] > lo && v[i] < hi;
      cand = in ? v[i] : cand;
      found = found || in;
    }
    const uint64_t has = __ballot(found);
    const int L = __builtin_ctzll(has);
    const uint64_t piv = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(cand >> 32), L) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((uint32_t)cand, L);
    int c = 0;
#pragma unroll
    for (int i = 0; i < kPfPL; ++i) c += __popcll(__ballot(lane + kWave * i < n && v[i] >= piv));
    if (c >= kk) {
      lo = piv;
      clo = c;
    } else {
      hi = piv;
    }
  }
  return lo;
}

// The same threshold as wave_threshold, usually in one pass: a 256-bin histogram (LDS, this
// wave's own bins) of the keys' scores over equal-width bins of [smin, smax], the highest bin B
// whose suffix count reaches kk, and th = the lowest key of the lowest score in bins >= B (that
// score in the high word, 0 in the low one). The bin of a score is monotone in the score, so
// #{key >= th} is that suffix count: at least kk, and at most kk + margin when bin B holds few
// enough keys; otherwise (and when every score is equal) the pivot search decides.
__device__ __forceinline__ uint64_t wave_threshold_hist(const uint64_t* buf, int n, int kk, int margin, uint32_t* hist) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t v[kPfPL];
  bool ok[kPfPL];
  uint32_t omx = 0, omn = ~0u;
#pragma unroll
  for (int i = 0; i < kPfPL; ++i) {
    ok[i] = lane + kWave * i < n;
    v[i] = buf[min(lane + kWave * i, kPfCap - 1)];
    const uint32_t o = (uint32_t)(v[i] >> 32);
    omx = ok[i] ? max(omx, o) : omx;
    omn = ok[i] ? min(omn, o) : omn;
  }
  omx = wave_max_u32(omx);
  omn = wave_min_u32(omn);
  const float s0 = ordered_to_score(omn);
  const float scale = (float)kPfHB / (ordered_to_score(omx) - s0);
  if (omx == omn || !(scale > 0.f && scale < INFINITY)) return wave_threshold(buf, n, kk, margin);
  *reinterpret_cast<uint4*>(&hist[4 * lane]) = make_uint4(0, 0, 0, 0);
  __builtin_amdgcn_wave_barrier();
  int bin[kPfPL];
#pragma unroll
  for (int i = 0; i < kPfPL; ++i) {
    bin[i] = min(kPfHB - 1, (int)((ordered_to_score((uint32_t)(v[i] >> 32)) - s0) * scale));
    if (ok[i]) atomicAdd(&hist[bin[i]], 1u);
  }
  __builtin_amdgcn_wave_barrier();
  const uint4 c = *reinterpret_cast<const uint4*>(&hist[4 * lane]);  // bins 4 lane .. 4 lane + 3
  const int tot = (int)(c.x + c.y + c.z + c.w);
  const int above = n - wave_incl_scan(tot);  // keys in the bins of higher lanes
  // suffix counts of the lane's bins, then the highest bin whose suffix count reaches kk
  const int g3 = above + (int)c.w, g2 = g3 + (int)c.z, g1 = g2 + (int)c.y, g0 = g1 + (int)c.x;
  const int jb = g3 >= kk ? 3 : (g2 >= kk ? 2 : (g1 >= kk ? 1 : (g0 >= kk ? 0 : -1)));
  const int mine = jb >= 0 ? 4 * lane + jb : -1;
  const int B = wave_reduce_i32(mine, [](int x, int y) { return max(x, y); });  // g0 of lane 0 is n >= kk
  const int gB = __builtin_amdgcn_readlane(jb == 3 ? g3 : (jb == 2 ? g2 : (jb == 1 ? g1 : g0)), B >> 2);
  __builtin_amdgcn_wave_barrier();
  if (gB > kk + margin) return wave_threshold(buf, n, kk, margin);
  uint32_t ts = ~0u;
#pragma unroll
  for (int i = 0; i < kPfPL; ++i) ts = ok[i] && bin[i] >= B ? min(ts, (uint32_t)(v[i] >> 32)) : ts;
  return (uint64_t)wave_min_u32(ts) << 32;
}

// Keeps the keys >= th of buf[0..n) at the front of buf (order not kept); returns their count.
__device__ int wave_compact_ge(uint64_t* buf, int n, uint64_t th) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t v[kPfPL];
#pragma unroll
  for (int i = 0; i < kPfPL; ++i) v[i] = lane + kWave * i < n ? buf[lane + kWave * i] : 0;
  __builtin_amdgcn_wave_barrier();
  const uint64_t lt = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int i = 0; i < kPfPL; ++i) {
    const bool p = lane + kWave * i < n && v[i] >= th;
    const uint64_t m = __ballot(p);
    if (p) buf[base + __popcll(m & lt)] = v[i];
    base += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  return base;
}

// ReLU of the four accumulator rows (an integer max on the bit pattern: negative floats, -0
// included, have a negative pattern), weighted by the head weights or, without them, summed
// (rows past H_I hold a zero query, so their ReLU is 0 either way).
template <bool HW>
__device__ __forceinline__ float head_sum(const f32x4& acc, const float* hw) {
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __int_as_float(max(__float_as_int(acc[i]), 0));
  if (HW) return fmaf(hw[3], r[3], fmaf(hw[2], r[2], fmaf(hw[1], r[1], hw[0] * r[0])));
  return (r[0] + r[1]) + (r[2] + r[3]);
}

// Appends the keys (score, e) of the lanes with `sel` that reach their query's threshold th to
// the candidate buffer of their query jq (of the QPT queries at buf[0..QPT)), which only this
// wave writes: slots by ballot rank after the wave-uniform count n[jq], which grows by the
// number appended. A wave whose lanes all miss the score floor thf skips the rest.
template <int QPT>
__device__ __forceinline__ void pf_append(uint64_t (*buf)[kPfCap], int (&n)[QPT], bool sel, int jq, float score,
                                          int e, float thf, uint64_t th) {
  const bool near = sel && score >= thf;
  if (__ballot(near) == 0) return;  // wave-uniform
  const uint64_t key = make_key(score, (uint32_t)e);
  const bool in = near && key >= th;
  const uint64_t below = (1ull << (threadIdx.x & (kWave - 1))) - 1ull;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const bool mine = in && jq == j;
    const uint64_t m = __ballot(mine);
    if (mine) buf[j][n[j] + __popcll(m & below)] = key;
    n[j] += __popcll(m);
  }
}

template <int KS, int QPT, bool HW>
__global__ __launch_bounds__(kPfNT) void index_block_kernel(IndexArgs a, int nqb) {
  constexpr int KT = PfTile<KS>::KT;
  constexpr int U = KT / 16 < kPfU ? KT / 16 : kPfU;  // groups per scoring step (divides KT / 16)
  static_assert((KT / 16) % U == 0 && U % 2 == 0, "whole, paired steps per tile");
  constexpr int RPQ = 16 / QPT;          // MFMA rows per query
  constexpr int QW = kPfRT * QPT;        // queries per wave
  constexpr int QB = kPfWaves * QW;      // queries per workgroup
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PfSmem<QB>& sm = *reinterpret_cast<PfSmem<QB>*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, col = lane & 15;
  const int b = blockIdx.x / nqb;
  const int qb = nqb - 1 - (blockIdx.x - b * nqb);  // the longest (causal) blocks start first
  const int t0 = qb * QB;
  const int chunk = blockIdx.y;
  const int kbytes = a.D_I >> 1, sbytes = a.D_I >> 5;
  const int pitch = kbytes + 16;
  const int kchunks = kbytes >> 4;       // 16-byte pieces per key

  if (tid < QB) {
    const int t = t0 + tid;
    sm.nv[tid] = t < a.T ? min(a.n_valid[(int64_t)b * a.T + t], a.N_cap) : 0;
  }
  // A operand: lane row `col` is query col / RPQ of the row tile, head col % RPQ
  uint4 qa[kPfRT][KS];
  int qs[kPfRT][KS];
  float hw[kPfRT][4];
#pragma unroll
  for (int rt = 0; rt < kPfRT; ++rt) {
    const int ta = t0 + wave * QW + rt * QPT + col / RPQ, ha = col % RPQ;
    const bool oka = ta < a.T && ha < a.H_I;
    const int64_t qrow = ((int64_t)b * a.T + ta) * a.H_I + ha;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bool okk = oka && (s * 128 + G * 32) < a.D_I;
      qa[rt][s] = okk ? *reinterpret_cast<const uint4*>(a.iq + qrow * kbytes + s * 64 + G * 16) : make_uint4(0, 0, 0, 0);
      qs[rt][s] = okk ? (int)a.iq_scale[qrow * sbytes + s * 4 + G] : 127;
    }
    // accumulator rows 4G + r: query (4G + r) / RPQ, head (4G + r) % RPQ
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * G + r;
      const int tr = t0 + wave * QW + rt * QPT + row / RPQ, hr = row % RPQ;
      hw[rt][r] = (tr < a.T && hr < a.H_I) ? (a.head_w ? a.head_w[((int64_t)b * a.T + tr) * a.H_I + hr] : 1.0f) : 0.0f;
    }
  }
  __syncthreads();
  // the query of this lane's scores within a row tile (QPT = 2: lane groups 0, 1 -> query 0,
  // groups 2, 3 -> query 1; QPT = 1: one query)
  const int jq = QPT == 2 ? (G >> 1) : 0;
  int nvq[kPfRT];
  int ncand[kPfRT][QPT] = {};  // candidates held by each of the wave's queries (wave-uniform)
  uint64_t th[kPfRT];
  float thf[kPfRT];  // the score of th (a key >= th has a score >= thf)
#pragma unroll
  for (int rt = 0; rt < kPfRT; ++rt) {
    nvq[rt] = sm.nv[wave * QW + rt * QPT + jq];
    th[rt] = 0;
    thf[rt] = -INFINITY;
  }
  int cmax = 0;
#pragma unroll 1
  for (int i = 0; i < QB; ++i) cmax = max(cmax, sm.nv[i]);
  const int c0 = chunk * a.chunk;
  const int c1 = min(c0 + a.chunk, cmax);
  const int n_tiles = c0 < c1 ? (c1 - c0 + KT - 1) / KT : 0;
  const uint8_t* ikb = a.ik + (int64_t)b * a.N_cap * kbytes;
  const uint8_t* iksb = a.ik_scale + (int64_t)b * a.N_cap * sbytes;

  // tile staging: each thread moves at most one piece of 16 code bytes and one scale byte
  static_assert(KT * 16 <= kPfNT * 16 && KT * (KS * 64) / 16 <= kPfNT, "one piece per thread");
  uint4 rv;
  uint8_t rs;
  const int key_c = tid / kchunks, part_c = tid - key_c * kchunks;
  const int key_s = tid / sbytes, part_s = tid - key_s * sbytes;
  auto tile_load = [&](int it) {
    const int e0 = c0 + it * KT;
    rv = tid < KT * kchunks ? ld_stream16(ikb + (int64_t)min(e0 + key_c, c1 - 1) * kbytes + 16 * part_c)
                            : make_uint4(0, 0, 0, 0);
    rs = tid < KT * sbytes ? iksb[(int64_t)min(e0 + key_s, c1 - 1) * sbytes + part_s] : (uint8_t)127;
  };
  auto tile_store = [&](int buf) {
    if (tid < KT * kchunks) *reinterpret_cast<uint4*>(&sm.kt[buf][key_c * pitch + 16 * part_c]) = rv;
    if (tid < KT * sbytes) sm.st[buf][tid] = rs;
  };
  if (n_tiles > 0) {
    tile_load(0);
    tile_store(0);
  }
  // every prologue load done here: otherwise the wait for the query operands, merged with the
  // loop's own loads at the loop head, becomes a wait for the next tile in every iteration
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll 1
  for (int it = 0; it < n_tiles; ++it) {
    const int cur = it & 1;
    if (it + 1 < n_tiles) tile_load(it + 1);
    const uint8_t* kt = sm.kt[cur];
    const uint8_t* st = sm.st[cur];
    const int e0 = c0 + it * KT;
    // U groups of 16 entries per step: their MFMAs issue back to back, then the scores
#pragma unroll 1
    for (int g = 0; g < KT / 16; g += U) {
      // every operand read (unconditional: a piece past D_I reads the row's first one, its scale
      // replaced by 1), then every product, then the scores: the MFMAs issue back to back and
      // the first results are ready when the score epilogue starts
      uint4 kv[U][KS];
      int ks[U][KS];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kl = 16 * (g + u) + col;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bool okk = (s * 128 + G * 32) < a.D_I;
          const int off = okk ? s * 64 + G * 16 : 0, soff = okk ? s * 4 + G : 0;
          kv[u][s] = *reinterpret_cast<const uint4*>(kt + kl * pitch + off);
          const int sv = st[kl * sbytes + soff];
          ks[u][s] = okk ? sv : 127;
        }
      }
      f32x4 acc[U][kPfRT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int rt = 0; rt < kPfRT; ++rt) {
          acc[u][rt] = mfma_fp4(qa[rt][0], kv[u][0], qs[rt][0], ks[u][0]);
#pragma unroll
          for (int s = 1; s < KS; ++s)
            acc[u][rt] = mfma_fp4_acc(qa[rt][s], kv[u][s], qs[rt][s], ks[u][s], acc[u][rt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (QPT == 2) {
        // lane group G holds rows 4G..4G+3: heads 0-3 / 4-7 of query 0 (G = 0, 1) and of query 1
        // (G = 2, 3). One permlane16 swap of the two groups' partial sums and one add leave
        // row 0 = group 0's query 0, row 1 = group 1's query 0, row 2 / 3 = query 1: every lane
        // then owns one (query, entry) score, query G >> 1 (= jq) and entry 16(g + (G & 1)) + col.
#pragma unroll
        for (int u = 0; u < U; u += 2) {
          const int e = e0 + 16 * (g + u + (G & 1)) + col;
#pragma unroll
          for (int rt = 0; rt < kPfRT; ++rt) {
            const float p0 = head_sum<HW>(acc[u][rt], hw[rt]), p1 = head_sum<HW>(acc[u + 1][rt], hw[rt]);
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
            const float part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            pf_append<QPT>(&sm.cand[wave * QW + rt * QPT], ncand[rt], e < nvq[rt], jq, part, e, thf[rt], th[rt]);
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = e0 + 16 * (g + u) + col;
#pragma unroll
          for (int rt = 0; rt < kPfRT; ++rt) {
            float part = head_sum<HW>(acc[u][rt], hw[rt]);
            part = add_xor32(add_xor16(part));
            pf_append<QPT>(&sm.cand[wave * QW + rt * QPT], ncand[rt], G == 0 && e < nvq[rt], 0, part, e, thf[rt], th[rt]);
          }
        }
      }
    }
    // reduce the wave's buffers that the next tile could overflow
#pragma unroll
    for (int rt = 0; rt < kPfRT; ++rt) {
#pragma unroll
      for (int j = 0; j < QPT; ++j) {
        const int q = wave * QW + rt * QPT + j;
        const int n = ncand[rt][j];
        if (n > kPfCap - KT) {
          const uint64_t kth = wave_threshold_hist(sm.cand[q], n, a.k, kPfMargin, sm.hist[wave]);
          const int m = wave_compact_ge(sm.cand[q], n, kth);
          ncand[rt][j] = m;
          if (jq == j) {
            th[rt] = kth;
            thf[rt] = ordered_to_score((uint32_t)(kth >> 32));
          }
        }
      }
    }
    if (it + 1 < n_tiles) tile_store(cur ^ 1);
    __syncthreads();
  }

  // the candidate counts go to nv (no longer read by any wave), each wave's own queries' slots,
  // read back below by the same wave (LDS requests of one wave complete in order)
  if (lane == 0) {
#pragma unroll
    for (int rt = 0; rt < kPfRT; ++rt)
#pragma unroll
      for (int j = 0; j < QPT; ++j) sm.nv[wave * QW + rt * QPT + j] = ncand[rt][j];
  }
  // final: each query's top min(k, candidates), ranked (one chunk) or as chunk winners
#pragma unroll 1
  for (int j = 0; j < QW; ++j) {
    const int q = wave * QW + j;
    const int t = t0 + q;
    if (t >= a.T) continue;
    const int64_t bq = (int64_t)b * a.T + t;
    uint64_t* buf = sm.cand[q];
    int n = __builtin_amdgcn_readfirstlane(sm.nv[q]);
    const int kk = min(a.k, n);
    if (n > kk + kPfMargin) n = wave_compact_ge(buf, n, wave_threshold_hist(buf, n, kk, kPfMargin, sm.hist[wave]));
    // rank the n (<= kk + margin) survivors; those ranked below kk are the answer
    uint64_t key[kPfRankPL];
    int rank[kPfRankPL];
#pragma unroll
    for (int i = 0; i < kPfRankPL; ++i) {
      key[i] = lane + kWave * i < n ? buf[lane + kWave * i] : 0;
      rank[i] = 0;
    }
    for (int j2 = 0; j2 < n; ++j2) {
      const uint64_t x = buf[j2];
#pragma unroll
      for (int i = 0; i < kPfRankPL; ++i) rank[i] += x > key[i];
    }
    if (a.n_chunks > 1) {
      uint64_t* out = a.part + (bq * a.n_chunks + chunk) * a.k;
#pragma unroll
      for (int i = 0; i < kPfRankPL; ++i)
        if (lane + kWave * i < n && rank[i] < kk) out[rank[i]] = key[i];
      for (int i = kk + lane; i < a.k; i += kWave) out[i] = 0;
      continue;
    }
    int32_t* oi = a.out_idx + bq * a.k;
    float* os = a.out_score ? a.out_score + bq * a.k : nullptr;
#pragma unroll
    for (int i = 0; i < kPfRankPL; ++i) {
      if (lane + kWave * i < n && rank[i] < kk) {
        oi[rank[i]] = (int32_t)(~(uint32_t)key[i]);
        if (os) os[rank[i]] = ordered_to_score((uint32_t)(key[i] >> 32));
      }
    }
    for (int i = kk + lane; i < a.k; i += kWave) {
      oi[i] = -1;
      if (os) os[i] = -INFINITY;
    }
  }
}

struct IndexPlan {
  int chunk, n_chunks, cap;
  size_t ws;
  bool decode;
  bool multi;    // decode of draft queries (kernel M)
  bool block;    // many-queries path (kernel P)
  int qpt, nqb;  // kernel P: queries per MFMA row tile, query blocks per sequence
};

static IndexPlan plan_index(int B, int T, int N_cap, int H_I, int D_I, int k) {
  IndexPlan p;
  p.block = false;
  p.qpt = 1;
  p.nqb = 0;
  // query-parallel path: at least ~1024 workgroups over the whole job; chunks of >= 1024
  // entries (multiples of 16) and no more than kMaxMergeKeys/k chunks per query
  const int max_chunks = kMaxMergeKeys / k > 0 ? kMaxMergeKeys / k : 1;
  const int64_t queries = (int64_t)B * T;
  int want = (int)((1024 + queries - 1) / queries);
  if (want < 1) want = 1;
  if (want > max_chunks) want = max_chunks;
  int chunk = (N_cap + want - 1) / want;
  if (chunk < 1024) chunk = 1024;
  chunk = (chunk + 15) & ~15;
  int n_chunks = (N_cap + chunk - 1) / chunk;
  if (n_chunks < 1) n_chunks = 1;
  while (n_chunks > max_chunks) {
    chunk *= 2;
    n_chunks = (N_cap + chunk - 1) / chunk;
  }
  p.chunk = chunk;
  p.n_chunks = n_chunks;
  p.cap = k <= 256 ? 512 : 2048;
  p.ws = (size_t)queries * n_chunks * k * sizeof(uint64_t);
  // decode path: few queries (at most one chunk workgroup per CU when they are alone)
  p.decode = k <= 1024 && queries <= 256;
  p.multi = p.decode && use_multi(B, T, H_I, D_I, k);
  if (p.decode) p.ws = p.multi ? multi_ws_bytes(B, T, N_cap, k) : decode_ws_bytes((int)queries, N_cap, k);
  // many queries: blocks of consecutive queries share the entry stream (kernel P); chunks of
  // the entries only when the query blocks alone leave the GPU idle (then the merge kernel)
  if (!p.decode && k <= kPfKMax) {
    p.block = true;
    p.qpt = H_I <= 8 ? 2 : 1;
    const int QB = kPfWaves * kPfRT * p.qpt;
    const int KT = D_I <= 128 ? PfTile<1>::KT : (D_I <= 256 ? PfTile<2>::KT : PfTile<4>::KT);
    p.nqb = (T + QB - 1) / QB;
    const int64_t nblk = (int64_t)B * p.nqb;
    int C = (int)((512 + nblk - 1) / nblk);
    const int cmax_merge = kMaxMergeKeys / k;
    if (C > cmax_merge) C = cmax_merge;
    const int cmax_size = (N_cap + 1023) / 1024;  // chunks of at least 1024 entries
    if (C > cmax_size) C = cmax_size;
    if (C < 1) C = 1;
    int chunk = (N_cap + C - 1) / C;
    chunk = (chunk + KT - 1) / KT * KT;
    p.chunk = chunk;
    p.n_chunks = (N_cap + chunk - 1) / chunk;
    if (p.n_chunks < 1) p.n_chunks = 1;
    p.cap = 512;
    p.ws = p.n_chunks > 1 ? (size_t)queries * p.n_chunks * k * sizeof(uint64_t) : 0;
  }
  return p;
}

template <int KS, int QPT>
static void launch_block_ks(const IndexArgs& a, int nqb, hipStream_t s) {
  constexpr int QB = kPfWaves * kPfRT * QPT;
  const size_t smem = sizeof(PfSmem<QB>);
  auto kern = a.head_w ? index_block_kernel<KS, QPT, true> : index_block_kernel<KS, QPT, false>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(kern, dim3(a.B * nqb, a.n_chunks), dim3(kPfNT), smem, s, a, nqb);
}

static int launch_block(const IndexArgs& a, const IndexPlan& p, int ks, hipStream_t s) {
  if (p.qpt == 2) {
    if (ks == 1) launch_block_ks<1, 2>(a, p.nqb, s);
    else if (ks == 2) launch_block_ks<2, 2>(a, p.nqb, s);
    else launch_block_ks<4, 2>(a, p.nqb, s);
  } else {
    if (ks == 1) launch_block_ks<1, 1>(a, p.nqb, s);
    else if (ks == 2) launch_block_ks<2, 1>(a, p.nqb, s);
    else launch_block_ks<4, 1>(a, p.nqb, s);
  }
  CSKV_LAUNCH_CHECK("csa_index_topk (query blocks)");
  if (p.n_chunks > 1) {
    const size_t smem = sizeof(Stage2Smem<512>);
    (void)hipFuncSetAttribute((const void*)index_merge_kernel<512>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)smem);
    hipLaunchKernelGGL(index_merge_kernel<512>, dim3(a.B * a.T), dim3(kIdxNT), smem, s, a);
  }
  return CSKV_OK;
}

template <int CAP, int KS>
static void launch_chunk(const IndexArgs& a, int queries, hipStream_t s) {
  const size_t smem = sizeof(Stage1Smem<CAP>);
  (void)hipFuncSetAttribute((const void*)index_chunk_kernel<CAP, KS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)smem);
  hipLaunchKernelGGL((index_chunk_kernel<CAP, KS>), dim3(queries, a.n_chunks), dim3(kIdxNT), smem, s, a);
}

template <int CAP>
static int launch_index(const IndexArgs& a, int queries, int ks, hipStream_t s) {
  if (ks == 1)
    launch_chunk<CAP, 1>(a, queries, s);
  else if (ks == 2)
    launch_chunk<CAP, 2>(a, queries, s);
  else
    launch_chunk<CAP, 4>(a, queries, s);
  CSKV_LAUNCH_CHECK("csa_index_topk (score)");
  const size_t smem = sizeof(Stage2Smem<CAP>);
  (void)hipFuncSetAttribute((const void*)index_merge_kernel<CAP>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(index_merge_kernel<CAP>, dim3(queries), dim3(kIdxNT), smem, s, a);
  return CSKV_OK;
}

}  // namespace cskv

using namespace cskv;

extern "C" CSKV_API size_t csa_index_topk_workspace_size(int B, int T, int N_cap, int H_I, int D_I, int k) {
  if (B < 1 || T < 1 || N_cap < 0 || k < 1 || k > 1024) return 0;
  return plan_index(B, T, N_cap > 0 ? N_cap : 1, H_I, D_I, k).ws;
}

extern "C" CSKV_API int csa_index_topk(const uint8_t* iq, const uint8_t* iq_scale, const float* head_w,
                                       const uint8_t* ik, const uint8_t* ik_scale, const int32_t* n_valid,
                                       int B, int T, int N_cap, int H_I, int D_I, int k, int32_t* out_idx,
                                       float* out_score, void* ws, size_t ws_bytes, void* stream) {
  CSKV_REQUIRE(B >= 1 && T >= 1 && N_cap >= 0, CSKV_EINVAL, "csa_index_topk: B=%d T=%d N_cap=%d", B, T, N_cap);
  CSKV_REQUIRE(D_I % 32 == 0 && D_I >= 32, CSKV_EINVAL, "csa_index_topk: D_I=%d must be a multiple of 32", D_I);
  CSKV_REQUIRE(D_I <= 512, CSKV_ENOTSUP, "csa_index_topk: D_I=%d > 512", D_I);
  CSKV_REQUIRE(H_I >= 1, CSKV_EINVAL, "csa_index_topk: H_I=%d", H_I);
  CSKV_REQUIRE(H_I <= 16, CSKV_ENOTSUP, "csa_index_topk: H_I=%d > 16", H_I);
  CSKV_REQUIRE(k >= 1, CSKV_EINVAL, "csa_index_topk: k=%d", k);
  CSKV_REQUIRE(k <= 1024, CSKV_ENOTSUP, "csa_index_topk: k=%d > 1024", k);
  CSKV_REQUIRE(iq && iq_scale && n_valid && out_idx, CSKV_EINVAL, "csa_index_topk: null pointer");
  CSKV_REQUIRE(N_cap == 0 || (ik && ik_scale), CSKV_EINVAL, "csa_index_topk: null key pointer");
  CSKV_REQUIRE(aligned16(iq) && (N_cap == 0 || aligned16(ik)), CSKV_EINVAL,
               "csa_index_topk: iq/ik must be 16-byte aligned");
  CSKV_REQUIRE(N_cap == 0 || (reinterpret_cast<uintptr_t>(ik_scale) & 3) == 0, CSKV_EINVAL,
               "csa_index_topk: ik_scale must be 4-byte aligned");
  const int Nc = N_cap > 0 ? N_cap : 1;
  IndexPlan p = plan_index(B, T, Nc, H_I, D_I, k);
  CSKV_REQUIRE(p.ws == 0 || (ws && ws_bytes >= p.ws), CSKV_EWORKSPACE, "csa_index_topk: workspace %zu < %zu bytes", ws_bytes,
               p.ws);
  CSKV_REQUIRE((int64_t)B * T < (1ll << 31), CSKV_ENOTSUP, "csa_index_topk: too many queries");
  IndexArgs a{iq, iq_scale, head_w, ik, ik_scale, n_valid, B, T, N_cap, H_I, D_I, k,
              p.chunk, p.n_chunks, reinterpret_cast<uint64_t*>(ws), out_idx, out_score};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int queries = B * T;
  const int ks = (D_I + 127) / 128;
  int rc = p.multi   ? launch_multi(a, ws, s)
           : p.decode ? launch_decode(a, queries, ks, ws, s)
           : p.block ? launch_block(a, p, ks, s)
                     : (p.cap == 512 ? launch_index<512>(a, queries, ks, s) : launch_index<2048>(a, queries, ks, s));
  if (rc != CSKV_OK) return rc;
  CSKV_LAUNCH_CHECK("csa_index_topk (merge)");
  return CSKV_OK;
}
