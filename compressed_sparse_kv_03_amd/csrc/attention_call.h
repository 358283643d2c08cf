// One hybrid_attn_decode / hybrid_attn_prefill call, as the two attention kernels take it:
// the 64-head kernel (attention.hip: long key sets, many queries) and the 16-head kernel
// (attention_g16.hip: a few hundred keys per query, few queries).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cskv {

enum { kKvBf16 = 0, kKvFp8 = 1, kKvMxfp4 = 2 };

struct AttnCall {
  const uint16_t* q;         // [nq, H, D]
  const int64_t* q_pos;      // [nq] (decode) or nullptr (prefill: pos0 + row)
  int64_t pos0;
  const void* ckv;           // [B_kv, N_cap, D] bf16 bits, fp8 codes, or MXFP4 codes [.., D/2]
  const void* ckv_scale;     // fp32 [B_kv, N_cap] (fp8) or E8M0 bytes [B_kv, N_cap, D/32] (MXFP4)
  int kv_dtype;              // kKvBf16, kKvFp8 or kKvMxfp4
  bool qk_fp4;               // MXFP4: QK^T on the scaled FP4 MFMA (64-head kernel; the 16-head one widens)
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
  uint16_t* out;             // [nq, H, d_v]
  float* out_lse;            // [nq, H]
  // decode with the state update: the step's new tokens are read from x_new (window positions
  // from the sequence's first query position on) and written to their ring slots by the call
  const uint16_t* x_new;     // [B, T, D] or nullptr (no append)
  const float* z_new;        // [B, T] or nullptr
  float* ring_z;             // [B, R] (with z_new)
};

// Window rows at or above kNewRow name row kNewRow + i of x_new (append mode); ring rows stay
// below it (B * R < kNewRow is checked by the call).
constexpr int kNewRow = 1 << 30;

// Append mode: the T new tokens of the sequence whose first query is qi (at position t0) go to
// ring slots (t0 + i) mod R, rows and pooling logits, with 16-byte vector stores by the nt
// threads of one workgroup. No workgroup of the call reads those slots: a query's window
// positions at or above t0 come from x_new, and the positions below t0 it sees
// (t0 + j - W + 1 .. t0 - 1) take other slots because R >= W + T - 1.
__device__ __forceinline__ void append_new_tokens(const uint16_t* __restrict__ x_new, const float* __restrict__ z_new,
                                                  uint16_t* __restrict__ ring_x, float* __restrict__ ring_z,
                                                  int qi, int T, int64_t t0, int R, int D, int tid, int nt) {
  const int b = qi / T;
  const int cpr = D >> 3;  // 16-byte chunks per row
  for (int c = tid; c < T * cpr; c += nt) {
    const int i = c / cpr, ch = c - i * cpr;
    const int64_t slot = (int64_t)b * R + (t0 + i) % R;
    const uint4 v = *reinterpret_cast<const uint4*>(x_new + (int64_t)(qi + i) * D + 8 * ch);
    *reinterpret_cast<uint4*>(ring_x + slot * D + 8 * ch) = v;
  }
  if (z_new && tid < T) ring_z[(int64_t)b * R + (t0 + tid) % R] = z_new[qi + tid];
}

namespace g16 {
size_t ws_bytes(int nq, int H, int d_v, int max_keys);
int launch(const char* name, const AttnCall& c, void* ws, size_t ws_bytes, hipStream_t s);
}  // namespace g16

}  // namespace cskv
