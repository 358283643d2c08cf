// Workgroup-wide exact top-k selection over distinct 64-bit keys held in LDS.
//
// Keys order the candidates of the lightning indexer: the high 32 bits are an
// order-preserving image of the fp32 score, the low 32 bits are ~index, so a
// larger key means (higher score, then lower index) and all keys of one query
// are distinct. Key 0 marks an empty slot and is never selected.
//
// Selection: find a threshold tau with kk <= #{key >= tau} <= CAP (first from
// a sorted sample of 256 keys, then by bisection on the key value, which ends
// because stepping tau changes the count by at most one), compact the keys >=
// tau into a CAP-sized buffer with wave-aggregated slots, and bitonic-sort that
// buffer in descending order. The top kk keys are then buf[0..kk).
#pragma once
#include "common.cuh"

namespace cskv {

__device__ __forceinline__ uint32_t score_to_ordered(float s) {
  s = s + 0.0f;  // -0 -> +0
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_to_score(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t make_key(float s, uint32_t idx) {
  return ((uint64_t)score_to_ordered(s) << 32) | (uint64_t)(~idx);
}

template <int NT>
__device__ __forceinline__ int block_sum_int(int v, int* red) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += red[i];
  return t;
}

// Descending bitonic sort of arr[0..P), P a power of two.
template <int NT>
__device__ void bitonic_sort_desc(uint64_t* arr, int P) {
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (P >> 1); i += NT) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const uint64_t a = arr[lo], b = arr[hi];
        const bool desc = (lo & size) == 0;
        if (desc ? (a < b) : (a > b)) {
          arr[lo] = b;
          arr[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

template <int NT>
__device__ int count_ge(const uint64_t* keys, int n, uint64_t tau, int* red) {
  int c = 0;
  for (int i = threadIdx.x; i < n; i += NT) c += keys[i] >= tau;
  return block_sum_int<NT>(c, red);
}

struct SelectScratch {
  uint64_t smp[256];
  int red[16];
  int cnt;
};

// Selects the kk largest keys of keys[0..n) (kk <= number of non-zero keys,
// kk <= CAP/2) into buf[0..kk) sorted descending. buf holds CAP entries.
// Must be called by all NT threads of the workgroup.
template <int NT, int CAP>
__device__ void select_topk(const uint64_t* keys, int n, int kk, uint64_t* buf, SelectScratch* sc) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t tau = 1;
  int c = count_ge<NT>(keys, n, tau, sc->red);
  if (c > CAP) {
    // sample-based first guess: about 2*kk + n/256 keys at or above tau
    for (int i = threadIdx.x; i < 256; i += NT) sc->smp[i] = keys[(int)(((int64_t)i * n) >> 8)];
    __syncthreads();
    bitonic_sort_desc<NT>(sc->smp, 256);
    int r = (int)(((int64_t)2 * kk * 256 + n - 1) / n);
    r = r < 1 ? 1 : (r > 255 ? 255 : r);
    uint64_t lo = 1, hi = ~0ull;  // count(lo) > CAP, count(hi) < kk (hi never tested: bound)
    uint64_t t = sc->smp[r];
    if (t == 0) t = 1;
    for (int it = 0; it < 160; ++it) {
      const int ct = count_ge<NT>(keys, n, t, sc->red);
      if (ct < kk) {
        hi = t;
      } else if (ct > CAP) {
        lo = t;
      } else {
        tau = t;
        c = ct;
        break;
      }
      t = lo + ((hi - lo) >> 1);
    }
  }
  // compact keys >= tau (c of them, kk <= c <= CAP)
  if (threadIdx.x == 0) sc->cnt = 0;
  __syncthreads();
  const int n_round = (n + NT - 1) / NT * NT;
  for (int i = threadIdx.x; i < n_round; i += NT) {
    const uint64_t key = i < n ? keys[i] : 0;
    const bool p = key >= tau;
    const uint64_t mask = __ballot(p);
    const int nw = __popcll(mask);
    int base = 0;
    if (lane == 0 && nw) base = atomicAdd(&sc->cnt, nw);
    base = __shfl(base, 0, kWave);
    const int off = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
    if (p && base + off < CAP) buf[base + off] = key;
  }
  __syncthreads();
  if (c > CAP) c = CAP;  // unreachable with distinct keys; keeps every write in bounds
  int P = 1;
  while (P < c) P <<= 1;
  for (int i = c + threadIdx.x; i < P; i += NT) buf[i] = 0;
  __syncthreads();
  bitonic_sort_desc<NT>(buf, P);
}

}  // namespace cskv
