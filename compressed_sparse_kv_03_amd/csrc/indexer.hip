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
  const int wave = threadIdx.x >> 6;
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
        acc += mfma_fp4(qa[s], kv[u][s], qs[s], sc);
      }
      // rows 4*kb + r are heads; ReLU, head weight, then sum over the 4 lane groups
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) part = fmaf(hw[r], fmaxf(acc[r], 0.f), part);
      part += __shfl_xor(part, 16, kWave);
      part += __shfl_xor(part, 32, kWave);
      const int el = (g0 + u) * 16 + col;
      sink(kb == 0 && el < n, el, make_key(part, (uint32_t)(e_begin + el)));
    }
    __builtin_amdgcn_wave_barrier();  // slot reads done before the next batch overwrites it
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
// Kernel P (one workgroup per query) scores a deterministic sample of the visible
// entries (S <= 2048: 128 runs of 16 consecutive entries spread evenly over them, or all
// of them when there are no more than 2048) and turns the j-th best sample key,
// j = ceil(8*k*S/n), into a lower bound L (the floor of its 20-bit score bin), so that
// about 8k keys of the query are >= L. Kernel A streams every chunk of entries once
// and keeps only the keys >= L: a chunk workgroup collects them in LDS and claims
// room in the query's candidate list with one atomic. Kernel C checks that at least
// k keys reached the list and that no chunk overflowed its buffer; then every key >= L
// is a candidate and the k-th best key is >= L, so the top-k of the candidates is the
// exact answer, found by rank selection. Otherwise (the sample overstated the top of
// the distribution, or very many keys tie at L) C recomputes the query exactly with a
// running top-k over all of its entries. The result is exact either way; only the
// time differs.
constexpr int kBins = 4096;       // 12-bit bins of the ordered score
constexpr int kSubBins = 256;     // next 8 bits
constexpr int kChunkA = 4096;     // entries per workgroup in kernel A
constexpr int kSampleMax = 2048;  // sampled entries per query
constexpr int kOver = 8;          // target candidates per query: kOver * k
constexpr int kCandWG = 1024;     // candidates one chunk workgroup may hold
constexpr int kCapF = 4096;       // candidates kernel C selects from directly
constexpr int kFinNT = 1024;      // threads of kernel C

struct DecodeArgs {
  IndexArgs a;
  uint64_t* cand;    // [Q][N_cap] candidate keys
  uint64_t* lbound;  // [Q] lower bound L
  uint32_t* cnt;     // [Q] candidates
  uint32_t* flag;    // [Q] nonzero: a chunk had more than kCandWG candidates
  int chunk, n_chunks;
};

__device__ __forceinline__ uint32_t key_bin(uint64_t key) { return (uint32_t)(key >> 52); }       // 12 bits
__device__ __forceinline__ uint32_t key_bin20(uint64_t key) { return (uint32_t)(key >> 44); }     // 20 bits

// Highest bin b (scanning from the top) whose cumulative count reaches kk; returns b and the
// count strictly above it in *above. NT is the block size (<= 1024); NB is a power of two.
// kk >= 1 and total >= kk. scratch holds at least 34 ints. Every thread must call it.
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
  int inc = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += v;
  }
  __syncthreads();
  if (lane == kWave - 1) scratch[w] = inc;
  if (t == 0) {  // defaults (bin 0) in case the counts do not reach kk
    scratch[32] = 0;
    scratch[33] = 0;
  }
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < w; ++i) wbase += scratch[i];
  const int incl = inc + wbase, excl = incl - s;
  __syncthreads();
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

// Wave-aggregated append of the keys passing `p` to dst[*cnt ...] (LDS counter); the
// counter keeps counting past cap so that overflow can be detected.
__device__ __forceinline__ void append_lds(bool p, uint64_t key, uint64_t* dst, int* cnt, int cap) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t mask = __ballot(p);
  if (mask == 0) return;
  const int nw = __popcll(mask);
  int base = 0;
  if (lane == 0) base = atomicAdd(cnt, nw);
  base = __shfl(base, 0, kWave);
  const int off = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
  if (p && base + off < cap) dst[base + off] = key;
}

constexpr int kSampNT = 1024;     // threads of kernel P

struct PSmem {
  uint64_t keys[kSampleMax];
  uint32_t hist[kBins];
  uint32_t sub[kSubBins];
  int scratch[34];
};

// Entry of sample i: all entries when nv <= kSampleMax (S = nv); else run i/16 of 128
// evenly spread runs of 16 consecutive entries (nv/128 >= 16, so the runs are disjoint).
__device__ __forceinline__ int sample_entry(int i, int nv, int S) {
  static_assert(kSampleMax == 128 * 16, "128 runs of 16 entries");
  return S == nv ? i : (int)(((int64_t)(i >> 4) * nv) >> 7) + (i & 15);
}

// Score the sampled entries of query q into keys[0..S).
// Every wave owns whole 16-sample groups and issues the loads of U groups before the
// first MFMA, so that the gathers overlap.
template <int KS>
__device__ void score_samples(const IndexArgs& a, int q, int nv, int S, const uint4* qa, const int* qs,
                              const float* hw, uint64_t* keys) {
  constexpr int U = KS == 1 ? 8 : (KS == 2 ? 4 : 2);
  constexpr int NW = kSampNT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int kb = lane >> 4, col = lane & 15;
  const int b = q / a.T;
  const int kbytes = a.D_I >> 1, sbytes = a.D_I >> 5;
  const uint8_t* ikb = a.ik + (int64_t)b * a.N_cap * kbytes;
  const uint8_t* iksb = a.ik_scale + (int64_t)b * a.N_cap * sbytes;
  const int groups = (S + 15) >> 4;
  for (int g0 = wave * U; g0 < groups; g0 += NW * U) {
    uint4 kv[U][KS];
    int sc[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = 16 * (g0 + u) + col;
      const int e = i < S ? sample_entry(i, nv, S) : 0;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kv[u][s] = make_uint4(0, 0, 0, 0);
        sc[u][s] = 127;
        if (i < S && (s * 128 + kb * 32) < a.D_I) {
          kv[u][s] = *reinterpret_cast<const uint4*>(ikb + (int64_t)e * kbytes + s * 64 + kb * 16);
          sc[u][s] = iksb[(int64_t)e * sbytes + s * 4 + kb];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = 16 * (g0 + u) + col;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc += mfma_fp4(qa[s], kv[u][s], qs[s], sc[u][s]);
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) part = fmaf(hw[r], fmaxf(acc[r], 0.f), part);
      part += __shfl_xor(part, 16, kWave);
      part += __shfl_xor(part, 32, kWave);
      if (kb == 0 && i < S) keys[i] = make_key(part, (uint32_t)sample_entry(i, nv, S));
    }
  }
}

template <int KS>
__global__ __launch_bounds__(kSampNT) void index_sample_kernel(DecodeArgs d) {
  __shared__ PSmem sm;
  const IndexArgs& a = d.a;
  const int q = blockIdx.x;
  const int nv = min(a.n_valid[q], a.N_cap);
  const int kk = min(a.k, nv);
  if (threadIdx.x == 0) {
    d.cnt[q] = 0;
    d.flag[q] = 0;
    d.lbound[q] = 1;  // below every key
  }
  if (kk == 0) return;
  const int S = min(nv, kSampleMax);
  int64_t jj = ((int64_t)kOver * kk * S + nv - 1) / nv;
  const int j = (int)(jj < 1 ? 1 : (jj > S ? S : jj));
  if (j >= S) return;  // the bound would admit (almost) everything: keep L = 1
  for (int i = threadIdx.x; i < kBins; i += kSampNT) sm.hist[i] = 0;
  for (int i = threadIdx.x; i < kSubBins; i += kSampNT) sm.sub[i] = 0;
  uint4 qa[KS];
  int qs[KS];
  float hw[4];
  load_query<KS>(a, q, qa, qs, hw);
  score_samples<KS>(a, q, nv, S, qa, qs, hw, sm.keys);
  __syncthreads();
  for (int i = threadIdx.x; i < S; i += kSampNT) atomicAdd(&sm.hist[key_bin(sm.keys[i])], 1u);
  __syncthreads();
  int above;
  const int bk = find_threshold_bin<kBins, kSampNT>(sm.hist, j, &above, sm.scratch);
  for (int i = threadIdx.x; i < S; i += kSampNT) {
    const uint32_t b20 = key_bin20(sm.keys[i]);
    if ((int)(b20 >> 8) == bk) atomicAdd(&sm.sub[b20 & 255], 1u);
  }
  __syncthreads();
  int above2;
  const int sk = find_threshold_bin<kSubBins, kSampNT>(sm.sub, j - above, &above2, sm.scratch);
  if (threadIdx.x == 0) {
    const uint64_t L = (uint64_t)(((uint32_t)bk << 8) | (uint32_t)sk) << 44;
    d.lbound[q] = L == 0 ? 1 : L;
  }
}

struct ASmem {
  uint64_t buf[kCandWG];
  __align__(16) uint8_t wsc[kIdxNT / kWave][1024];
  int cnt;
  int base;
};

template <int KS>
__global__ __launch_bounds__(kIdxNT) void index_filter_kernel(DecodeArgs d) {
  __shared__ ASmem sm;
  const IndexArgs& a = d.a;
  const int q = blockIdx.x;
  const int b = q / a.T;
  const int nv = min(a.n_valid[q], a.N_cap);
  const int c0 = blockIdx.y * d.chunk;
  const int c1 = min(c0 + d.chunk, nv);
  if (c0 >= c1) return;
  if (threadIdx.x == 0) sm.cnt = 0;
  const uint64_t L = d.lbound[q];
  uint4 qa[KS];
  int qs[KS];
  float hw[4];
  load_query<KS>(a, q, qa, qs, hw);
  __syncthreads();
  uint64_t* buf = sm.buf;
  int* cnt = &sm.cnt;
  score_range_to<KS, kIdxNT>(a, b, c0, c1, qa, qs, hw, sm.wsc[threadIdx.x >> 6],
                             [buf, cnt, L](bool p, int, uint64_t key) { append_lds(p && key >= L, key, buf, cnt, kCandWG); });
  __syncthreads();
  const int c = sm.cnt;
  if (c == 0) return;
  if (c > kCandWG) {
    if (threadIdx.x == 0) atomicOr(&d.flag[q], 1u);
    return;
  }
  if (threadIdx.x == 0) sm.base = (int)atomicAdd(&d.cnt[q], (uint32_t)c);
  __syncthreads();
  const int base = sm.base;
  uint64_t* dst = d.cand + (int64_t)q * a.N_cap;
  for (int i = threadIdx.x; i < c; i += kIdxNT)
    if (base + i < a.N_cap) dst[base + i] = sm.buf[i];
}

struct CSmem {
  uint64_t buf[kCapF];
  uint64_t keys[1024 + kSub];  // exact paths: running winners + one sub-chunk
  __align__(16) uint8_t wsc[kFinNT / kWave][1024];
  uint32_t hist[kBins];
  SelectScratch sc;
  int scratch[34];
  unsigned long long mx;
  int cnt;
};

__device__ __forceinline__ void write_key(const IndexArgs& a, int32_t* oi, float* os, int slot, uint64_t key) {
  oi[slot] = (int32_t)(~(uint32_t)key);
  if (os) os[slot] = ordered_to_score((uint32_t)(key >> 32));
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

template <int KS>
__global__ __launch_bounds__(kFinNT) void index_final_kernel(DecodeArgs d) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  CSmem& sm = *reinterpret_cast<CSmem*>(smem_raw);
  const IndexArgs& a = d.a;
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int nv = min(a.n_valid[q], a.N_cap);
  const int kk = min(a.k, nv);
  int32_t* oi = a.out_idx + (int64_t)q * a.k;
  float* os = a.out_score ? a.out_score + (int64_t)q * a.k : nullptr;
  for (int i = kk + tid; i < a.k; i += kFinNT) {  // padding
    oi[i] = -1;
    if (os) os[i] = -INFINITY;
  }
  if (kk == 0) return;
  const int n_cand = min((int)d.cnt[q], a.N_cap);
  const bool exact_ok = d.flag[q] == 0 && n_cand >= kk;
  const uint64_t* cq = d.cand + (int64_t)q * a.N_cap;
  if (exact_ok && n_cand <= kCapF) {
    // Histogram of (key - L) over 4096 bins spanning [L, max key]; the bin holding the k-th
    // best key and every bin above it form a set S' that holds the top-k, and a key of S'
    // is beaten only by keys of S', so its rank within S' is its final slot.
    const uint64_t L = d.lbound[q];
    if (tid == 0) {
      sm.mx = 0;
      sm.cnt = 0;
    }
    uint64_t mx = 0;
    for (int i = tid; i < kBins; i += kFinNT) sm.hist[i] = 0;
    for (int i = tid; i < n_cand; i += kFinNT) {
      const uint64_t v = cq[i];
      sm.buf[i] = v;
      mx = v > mx ? v : mx;
    }
    mx = wave_max_u64(mx);
    __syncthreads();
    if ((tid & (kWave - 1)) == 0) atomicMax(&sm.mx, (unsigned long long)mx);
    __syncthreads();
    const uint64_t R = sm.mx - L;
    const int shift = R == 0 ? 0 : max(0, 64 - __builtin_clzll(R) - 12);
    for (int i = tid; i < n_cand; i += kFinNT) atomicAdd(&sm.hist[(sm.buf[i] - L) >> shift], 1u);
    __syncthreads();
    int above;
    const uint32_t thr = (uint32_t)find_threshold_bin<kBins, kFinNT>(sm.hist, kk, &above, sm.scratch);
    for (int i0 = 0; i0 < n_cand; i0 += kFinNT) {
      const int i = i0 + tid;
      const uint64_t key = i < n_cand ? sm.buf[i] : 0;
      append_lds(i < n_cand && ((key - L) >> shift) >= thr, key, sm.keys, &sm.cnt, kCapF);
    }
    __syncthreads();
    const int m = min(sm.cnt, kCapF);
    for (int i = tid; i < m; i += kFinNT) {
      const uint64_t key = sm.keys[i];
      int rank = 0;
      for (int jx = 0; jx < m; ++jx) rank += sm.keys[jx] > key;
      if (rank < kk) write_key(a, oi, os, rank, key);
    }
    return;
  }
  // running top-k: over the candidate list (exact_ok), else over every visible entry
  uint4 qa[KS];
  int qs[KS];
  float hw[4];
  if (!exact_ok) load_query<KS>(a, q, qa, qs, hw);
  const int total = exact_ok ? n_cand : nv;
  int kept = 0;
  for (int s0 = 0; s0 < total; s0 += kSub) {
    const int s1 = min(s0 + kSub, total);
    if (exact_ok) {
      for (int i = threadIdx.x; i < s1 - s0; i += kFinNT) sm.keys[kept + i] = cq[s0 + i];
    } else {
      score_range<KS, kFinNT, 2>(a, q / a.T, s0, s1, qa, qs, hw, sm.keys + kept, sm.wsc[threadIdx.x >> 6]);
    }
    __syncthreads();
    const int nn = kept + (s1 - s0);
    const int k2 = min(kk, nn);
    select_topk<kFinNT, kCapF>(sm.keys, nn, k2, sm.buf, &sm.sc);
    for (int i = threadIdx.x; i < k2; i += kFinNT) sm.keys[i] = sm.buf[i];
    __syncthreads();
    kept = k2;
  }
  for (int i = threadIdx.x; i < kept; i += kFinNT) write_key(a, oi, os, i, sm.keys[i]);
}

static int decode_chunks(int N_cap) { return (N_cap + kChunkA - 1) / kChunkA; }

static size_t decode_ws_bytes(int queries, int N_cap) {
  return (size_t)queries * N_cap * sizeof(uint64_t) + (size_t)queries * (sizeof(uint64_t) + 2 * sizeof(uint32_t));
}

template <int KS>
static void launch_decode_ks(const DecodeArgs& d, int queries, hipStream_t s) {
  hipLaunchKernelGGL((index_sample_kernel<KS>), dim3(queries), dim3(kSampNT), 0, s, d);
  if (d.n_chunks > 0) hipLaunchKernelGGL((index_filter_kernel<KS>), dim3(queries, d.n_chunks), dim3(kIdxNT), 0, s, d);
  const size_t smem = sizeof(CSmem);
  (void)hipFuncSetAttribute((const void*)index_final_kernel<KS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
  hipLaunchKernelGGL((index_final_kernel<KS>), dim3(queries), dim3(kFinNT), smem, s, d);
}

static int launch_decode(const IndexArgs& a, int queries, int ks, void* ws, hipStream_t s) {
  DecodeArgs d;
  d.a = a;
  d.chunk = kChunkA;
  d.n_chunks = decode_chunks(a.N_cap);
  unsigned char* w = reinterpret_cast<unsigned char*>(ws);
  d.cand = reinterpret_cast<uint64_t*>(w);
  w += (size_t)queries * a.N_cap * sizeof(uint64_t);
  d.lbound = reinterpret_cast<uint64_t*>(w);
  w += (size_t)queries * sizeof(uint64_t);
  d.cnt = reinterpret_cast<uint32_t*>(w);
  w += (size_t)queries * sizeof(uint32_t);
  d.flag = reinterpret_cast<uint32_t*>(w);
  if (ks == 1)
    launch_decode_ks<1>(d, queries, s);
  else if (ks == 2)
    launch_decode_ks<2>(d, queries, s);
  else
    launch_decode_ks<4>(d, queries, s);
  CSKV_LAUNCH_CHECK("csa_index_topk (decode)");
  return CSKV_OK;
}

struct IndexPlan {
  int chunk, n_chunks, cap;
  size_t ws;
  bool decode;
};

static IndexPlan plan_index(int B, int T, int N_cap, int k) {
  IndexPlan p;
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
  // decode path: few queries (candidate lists of N_cap keys per query stay small)
  p.decode = k <= 1024 && (size_t)queries * N_cap <= ((size_t)1 << 26);
  if (p.decode) p.ws = decode_ws_bytes((int)queries, N_cap);
  return p;
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
  (void)H_I;
  (void)D_I;
  if (B < 1 || T < 1 || N_cap < 0 || k < 1 || k > 1024) return 0;
  return plan_index(B, T, N_cap > 0 ? N_cap : 1, k).ws;
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
  const int Nc = N_cap > 0 ? N_cap : 1;
  IndexPlan p = plan_index(B, T, Nc, k);
  CSKV_REQUIRE(ws && ws_bytes >= p.ws, CSKV_EWORKSPACE, "csa_index_topk: workspace %zu < %zu bytes", ws_bytes,
               p.ws);
  CSKV_REQUIRE((int64_t)B * T < (1ll << 31), CSKV_ENOTSUP, "csa_index_topk: too many queries");
  IndexArgs a{iq, iq_scale, head_w, ik, ik_scale, n_valid, B, T, N_cap, H_I, D_I, k,
              p.chunk, p.n_chunks, reinterpret_cast<uint64_t*>(ws), out_idx, out_score};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int queries = B * T;
  const int ks = (D_I + 127) / 128;
  int rc = p.decode ? launch_decode(a, queries, ks, ws, s)
                    : (p.cap == 512 ? launch_index<512>(a, queries, ks, s) : launch_index<2048>(a, queries, ks, s));
  if (rc != CSKV_OK) return rc;
  CSKV_LAUNCH_CHECK("csa_index_topk (merge)");
  return CSKV_OK;
}
