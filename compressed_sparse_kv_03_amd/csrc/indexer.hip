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
};

// Score entries [e_begin, e_end) of one query into keys[0..e_end-e_begin), 16 per wave step.
// KS = number of 128-wide k steps (D_I <= 128 * KS); U = 16-entry groups in flight per wave.
template <int KS>
__device__ __forceinline__ void score_range(const IndexArgs& a, int b, int e_begin, int e_end,
                                            const uint4* qa, const int* qs, const float* hw,
                                            uint64_t* keys) {
  constexpr int U = KS == 1 ? 16 : (KS == 2 ? 8 : 4);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int kb = lane >> 4, col = lane & 15;
  const int kbytes = a.D_I >> 1, sbytes = a.D_I >> 5;
  const uint8_t* ikb = a.ik + (int64_t)b * a.N_cap * kbytes;
  const uint8_t* iksb = a.ik_scale + (int64_t)b * a.N_cap * sbytes;
  const int n = e_end - e_begin;
  const int groups = (n + 15) >> 4;
  for (int g0 = wave * U; g0 < groups; g0 += (kIdxNT / kWave) * U) {
    uint4 kv[U][KS];
    int ks[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e_begin + (g0 + u) * 16 + col;
      const bool ok = (g0 + u) < groups && e < e_end;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kv[u][s] = make_uint4(0, 0, 0, 0);
        ks[u][s] = 127;
        if (ok && (s * 128 + kb * 32) < a.D_I) {
          kv[u][s] = *reinterpret_cast<const uint4*>(ikb + (int64_t)e * kbytes + s * 64 + kb * 16);
          ks[u][s] = iksb[(int64_t)e * sbytes + s * 4 + kb];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u >= groups) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc += mfma_fp4(qa[s], kv[u][s], qs[s], ks[u][s]);
      // rows 4*kb + r are heads; ReLU, head weight, then sum over the 4 lane groups
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) part = fmaf(hw[r], fmaxf(acc[r], 0.f), part);
      part += __shfl_xor(part, 16, kWave);
      part += __shfl_xor(part, 32, kWave);
      const int el = (g0 + u) * 16 + col;
      if (kb == 0 && el < n) keys[el] = make_key(part, (uint32_t)(e_begin + el));
    }
  }
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
    score_range<KS>(a, b, s0, s1, qa, qs, hw, sm.keys + kept);
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
// Kernel Z zeroes each query's candidate counter and 12-bit histogram. Kernel A
// gives each (query, chunk of entries) one workgroup: it scores the chunk into
// LDS, finds the chunk's local top-k threshold with two LDS histograms (12 bits
// of the ordered score, then the next 8 bits inside the threshold bin), claims
// room for exactly the keys at or above it with one atomic on the query's
// counter, writes them contiguously to the query's candidate list and adds
// their 12-bit bin counts to the query's histogram. Kernel C, one workgroup per
// query, finds the highest bin b' whose cumulative count from the top reaches k,
// keeps the candidates in bins >= b' (a few hundred) and sorts them.
// Exactness: every global top-k key is in its chunk's top-k, so it is a
// candidate; the candidates in bins >= b' therefore include the whole global
// top-k, and b' is the bin of the k-th best key (were it higher, k candidates
// would beat that key).
constexpr int kBins = 4096;     // 12-bit bins of the ordered score
constexpr int kSubBins = 256;   // next 8 bits
constexpr int kChunkA = 4096;   // entries per workgroup in kernel A
constexpr int kCapF = 2048;     // candidates kernel C sorts directly

struct DecodeArgs {
  IndexArgs a;
  uint64_t* cand;   // [Q][N_cap] candidate keys
  uint32_t* hist;   // [Q][kBins] 12-bit bin counts of the candidates
  uint32_t* cnt;    // [Q] candidates
  int chunk, n_chunks;
};

__device__ __forceinline__ uint32_t key_bin(uint64_t key) { return (uint32_t)(key >> 52); }       // 12 bits
__device__ __forceinline__ uint32_t key_bin20(uint64_t key) { return (uint32_t)(key >> 44); }     // 20 bits

// Highest bin b (scanning from the top) whose cumulative count reaches kk; returns b and the
// count strictly above it in *above. NB is a multiple of NT. kk >= 1 and total >= kk.
// scratch holds at least 34 ints.
template <int NB, int NT = kIdxNT>
__device__ int find_threshold_bin(const uint32_t* hist, int kk, int* above, int* scratch) {
  constexpr int PER = NB / NT;
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t >> 6;
  // thread t owns bins [NB - PER*(t+1), NB - PER*t), i.e. the t-th slice from the top
  const int top = NB - PER * t;
  int s = 0;
#pragma unroll
  for (int i = 1; i <= PER; ++i) s += hist[top - i];
  int inc = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += v;
  }
  __syncthreads();
  if (lane == kWave - 1) scratch[w] = inc;
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < w; ++i) wbase += scratch[i];
  const int incl = inc + wbase, excl = incl - s;
  __syncthreads();
  if (excl < kk && incl >= kk) {
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

// Wave-aggregated append of the keys passing `p` to dst[*cnt ...] (LDS counter).
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

__global__ __launch_bounds__(kIdxNT) void index_zero_kernel(DecodeArgs d) {
  const int q = blockIdx.x;
  uint32_t* h = d.hist + (int64_t)q * kBins;
  for (int i = threadIdx.x; i < kBins; i += kIdxNT) h[i] = 0;
  if (threadIdx.x == 0) d.cnt[q] = 0;
}

struct ASmem {
  uint64_t keys[kChunkA];
  uint32_t hist[kBins];
  uint32_t sub[kSubBins];
  int scratch[34];
  int cnt;
  int base;
};

template <int KS>
__global__ __launch_bounds__(kIdxNT) void index_score_kernel(DecodeArgs d) {
  __shared__ ASmem sm;
  const IndexArgs& a = d.a;
  const int q = blockIdx.x;
  const int b = q / a.T;
  const int nv = min(a.n_valid[q], a.N_cap);
  const int chunk = blockIdx.y;
  const int c0 = chunk * d.chunk;
  const int c1 = min(c0 + d.chunk, nv);
  if (c0 >= c1) return;
  const int n = c1 - c0;
  for (int i = threadIdx.x; i < kBins; i += kIdxNT) sm.hist[i] = 0;
  for (int i = threadIdx.x; i < kSubBins; i += kIdxNT) sm.sub[i] = 0;
  if (threadIdx.x == 0) sm.cnt = 0;
  uint4 qa[KS];
  int qs[KS];
  float hw[4];
  load_query<KS>(a, q, qa, qs, hw);
  __syncthreads();
  score_range<KS>(a, b, c0, c1, qa, qs, hw, sm.keys);
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kIdxNT) atomicAdd(&sm.hist[key_bin(sm.keys[i])], 1u);
  __syncthreads();
  const int kk = min(a.k, n);
  int above;
  const int bk = find_threshold_bin<kBins>(sm.hist, kk, &above, sm.scratch);
  for (int i = threadIdx.x; i < n; i += kIdxNT) {
    const uint32_t b20 = key_bin20(sm.keys[i]);
    if ((int)(b20 >> 8) == bk) atomicAdd(&sm.sub[b20 & 255], 1u);
  }
  __syncthreads();
  int above2;
  const int sk = find_threshold_bin<kSubBins>(sm.sub, kk - above, &above2, sm.scratch);
  const uint32_t thr20 = ((uint32_t)bk << 8) | (uint32_t)sk;
  // keys at or above the threshold: the bins above bk, plus sub-bins >= sk of bin bk
  const int n_keep = above + above2 + (int)sm.sub[sk];
  if (threadIdx.x == 0) sm.base = (int)atomicAdd(&d.cnt[q], (uint32_t)n_keep);
  for (int i = threadIdx.x; i < kBins; i += kIdxNT) sm.hist[i] = 0;
  __syncthreads();
  uint64_t* cand = d.cand + (int64_t)q * a.N_cap + sm.base;
  const int n_round = (n + kIdxNT - 1) / kIdxNT * kIdxNT;
  for (int i = threadIdx.x; i < n_round; i += kIdxNT) {
    const uint64_t key = i < n ? sm.keys[i] : 0;
    const bool p = i < n && key_bin20(key) >= thr20;
    append_lds(p, key, cand, &sm.cnt, n_keep);
    if (p) atomicAdd(&sm.hist[key_bin(key)], 1u);
  }
  __syncthreads();
  uint32_t* gh = d.hist + (int64_t)q * kBins;
  for (int i = threadIdx.x; i < kBins; i += kIdxNT) {
    const uint32_t c = sm.hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

constexpr int kFinNT = 1024;   // threads of the final per-query kernel

struct CSmem {
  uint32_t hist[kBins];
  uint64_t buf[kCapF];
  uint64_t keys[1024 + kSub];  // slow path: running winners + one sub-chunk
  SelectScratch sc;
  int scratch[34];
  int cnt;
};

__global__ __launch_bounds__(kFinNT) void index_final_kernel(DecodeArgs d) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  CSmem& sm = *reinterpret_cast<CSmem*>(smem_raw);
  const IndexArgs& a = d.a;
  const int q = blockIdx.x;
  const int nv = min(a.n_valid[q], a.N_cap);
  const int kk = min(a.k, nv);
  int32_t* oi = a.out_idx + (int64_t)q * a.k;
  float* os = a.out_score ? a.out_score + (int64_t)q * a.k : nullptr;
  // slots >= kk are padding
  for (int i = kk + threadIdx.x; i < a.k; i += kFinNT) {
    oi[i] = -1;
    if (os) os[i] = -INFINITY;
  }
  if (kk == 0) return;
  const uint32_t* gh = d.hist + (int64_t)q * kBins;
  for (int i = threadIdx.x; i < kBins; i += kFinNT) sm.hist[i] = gh[i];
  __syncthreads();
  int above;
  const int bp = find_threshold_bin<kBins, kFinNT>(sm.hist, kk, &above, sm.scratch);
  int cstar = 0;
  for (int i = threadIdx.x; i < kBins; i += kFinNT) cstar += i >= bp ? (int)sm.hist[i] : 0;
  cstar = block_sum_int<kFinNT>(cstar, sm.sc.red);
  const int n_cand = min((int)d.cnt[q], a.N_cap);
  const uint64_t* cq = d.cand + (int64_t)q * a.N_cap;
  if (cstar <= kCapF) {
    if (threadIdx.x == 0) sm.cnt = 0;
    __syncthreads();
    constexpr int U = 4;  // independent loads in flight per thread
    for (int i0 = 0; i0 < n_cand; i0 += U * kFinNT) {
      uint64_t kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kFinNT + threadIdx.x;
        kv[u] = i < n_cand ? cq[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kFinNT + threadIdx.x;
        append_lds(i < n_cand && (int)key_bin(kv[u]) >= bp, kv[u], sm.buf, &sm.cnt, kCapF);
      }
    }
    __syncthreads();
    // rank selection: keys are distinct, so key i goes to slot #{keys greater than it}
    const int c = min(sm.cnt, kCapF);
    for (int i = threadIdx.x; i < c; i += kFinNT) {
      const uint64_t key = sm.buf[i];
      int rank = 0;
      for (int j = 0; j < c; ++j) rank += sm.buf[j] > key;
      if (rank < kk) {
        oi[rank] = (int32_t)(~(uint32_t)key);
        if (os) os[rank] = ordered_to_score((uint32_t)(key >> 32));
      }
    }
    return;
  }
  // many keys tie into the threshold bin: exact running top-k over the filtered candidates
  int kept = 0;
  for (int s0 = 0; s0 < n_cand; s0 += kSub) {
    const int s1 = min(s0 + kSub, n_cand);
    if (threadIdx.x == 0) sm.cnt = 0;
    __syncthreads();
    const int n_round = (s1 - s0 + kFinNT - 1) / kFinNT * kFinNT;
    for (int i = threadIdx.x; i < n_round; i += kFinNT) {
      const int j = s0 + i;
      const uint64_t key = j < s1 ? cq[j] : 0;
      append_lds(j < s1 && (int)key_bin(key) >= bp, key, sm.keys + kept, &sm.cnt, kSub);
    }
    __syncthreads();
    const int nn = kept + sm.cnt;
    if (nn > 0) {
      const int k2 = min(kk, nn);
      select_topk<kFinNT, kCapF>(sm.keys, nn, k2, sm.buf, &sm.sc);
      for (int i = threadIdx.x; i < k2; i += kFinNT) sm.keys[i] = sm.buf[i];
      __syncthreads();
      kept = k2;
    }
  }
  for (int i = threadIdx.x; i < kept; i += kFinNT) {
    const uint64_t key = sm.keys[i];
    oi[i] = (int32_t)(~(uint32_t)key);
    if (os) os[i] = ordered_to_score((uint32_t)(key >> 32));
  }
}

static int decode_chunks(int N_cap) { return (N_cap + kChunkA - 1) / kChunkA; }

static size_t decode_ws_bytes(int queries, int N_cap) {
  return (size_t)queries * N_cap * sizeof(uint64_t) + (size_t)queries * (kBins + 1) * sizeof(uint32_t);
}

struct IndexPlan {
  int chunk, n_chunks, cap;
  size_t ws;
  bool decode;
};

static IndexPlan plan_index(int B, int T, int N_cap, int k) {
  IndexPlan p;
  // at least ~1024 workgroups over the whole job; chunks of >= 1024 entries
  // (multiples of 16) and no more than kMaxMergeKeys/k chunks per query
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

template <int KS>
static void launch_decode_score(const DecodeArgs& d, int queries, int n_chunks, hipStream_t s) {
  hipLaunchKernelGGL((index_score_kernel<KS>), dim3(queries, n_chunks), dim3(kIdxNT), 0, s, d);
}

static int launch_decode(const IndexArgs& a, int queries, int ks, void* ws, hipStream_t s) {
  DecodeArgs d;
  d.a = a;
  d.chunk = kChunkA;
  d.n_chunks = decode_chunks(a.N_cap);
  unsigned char* w = reinterpret_cast<unsigned char*>(ws);
  d.cand = reinterpret_cast<uint64_t*>(w);
  w += (size_t)queries * a.N_cap * sizeof(uint64_t);
  d.hist = reinterpret_cast<uint32_t*>(w);
  w += (size_t)queries * kBins * sizeof(uint32_t);
  d.cnt = reinterpret_cast<uint32_t*>(w);
  hipLaunchKernelGGL(index_zero_kernel, dim3(queries), dim3(kIdxNT), 0, s, d);
  CSKV_LAUNCH_CHECK("csa_index_topk (zero)");
  if (d.n_chunks > 0) {
    if (ks == 1)
      launch_decode_score<1>(d, queries, d.n_chunks, s);
    else if (ks == 2)
      launch_decode_score<2>(d, queries, d.n_chunks, s);
    else
      launch_decode_score<4>(d, queries, d.n_chunks, s);
    CSKV_LAUNCH_CHECK("csa_index_topk (score)");
  }
  const size_t smem = sizeof(CSmem);
  (void)hipFuncSetAttribute((const void*)index_final_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(index_final_kernel, dim3(queries), dim3(kFinNT), smem, s, d);
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
