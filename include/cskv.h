/*
 * cskv.h - C ABI of the MI355X (gfx950) hybrid compressed attention library.
 *
 * The method (DeepSeek-V4 hybrid attention) is described on the page
 * "DeepSeek-V4가 이차적 어텐션 비용 없이 백만 토큰 컨텍스트를 달성하는 방법",
 * section "두 가지 압축 전략: CSA 및 HCA": Compressed Sparse Attention (CSA)
 * softmax-pools every 4 consecutive tokens into one KV entry, an FP4
 * "lightning indexer" scores the entries and keeps the top-k (about 128), and
 * attention runs over those plus a sliding window; Heavily Compressed
 * Attention (HCA) pools 128 tokens per entry and attends to all entries; both
 * use MQA (one shared KV head) with partial RoPE. The page "딥시크 V4 분석:
 * CSA·HCA 어텐션으로 100만 토큰 컨텍스트를 저비용에 구현한 방법", section
 * "쉽게 이해하기", gives the 128-token window branch.
 *
 * Conventions shared by every call
 *  - Tensor arguments are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or keeps a pointer after a call returns.
 *  - Every call is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and never synchronises. Errors found while validating arguments are
 *    returned before anything is enqueued; a failed launch returns CSKV_EHIP.
 *  - Layouts are dense row-major unless a stride argument says otherwise.
 *    bf16 values are passed as uint16_t bit patterns. fp8 is OCP e4m3fn.
 *    MXFP4 is OCP MX FP4: e2m1 codes packed two per byte, element 2i in the
 *    low nibble of byte i, with one E8M0 scale byte (2^(E-127)) per 32 elements.
 *  - All base pointers must be 16-byte aligned.
 *  - The library holds no mutable global state; calls are thread-safe.
 *    Calls that write the same buffers must be ordered by the caller.
 *  - cskv_last_error() returns a thread-local message for the last failure.
 */
#ifndef CSKV_H_
#define CSKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSKV_ABI_VERSION 3

#if defined(__GNUC__)
#define CSKV_API __attribute__((visibility("default")))
#else
#define CSKV_API
#endif

/* Return codes. */
#define CSKV_OK 0
#define CSKV_EINVAL (-1)    /* null pointer, bad dimension, misalignment */
#define CSKV_ENOTSUP (-2)   /* a shape outside what the kernels support */
#define CSKV_EWORKSPACE (-3) /* workspace missing or too small */
#define CSKV_EHIP (-4)      /* a HIP launch failed */

/* Storage dtypes of compressed entries. */
#define CSKV_BF16 0
#define CSKV_FP8_E4M3 1
#define CSKV_MXFP4 2   /* OCP MXFP4: e2m1 codes [.., D/2] (element 2i in the low nibble) + E8M0 [.., D/32] */
/* Flag OR-ed into the ckv_dtype CSKV_MXFP4 of hybrid_attn_decode(_noalloc) and
 * hybrid_attn_prefill (D % 64 == 0): the 64-head kernel takes the entry logits q . key on the
 * scaled FP4 x FP8 MFMA straight from the stored e2m1 codes and E8M0 exponents, the rotated
 * query held as a sum of e4m3 parts with one power-of-two scale per 64 dims (the mixed-precision
 * matrix cores of CDNA4, for the FP4 main KV of the "SWA Bounded Replay" global attention state;
 * without the flag the entries are widened exactly to bf16 first). Parts: two per raw dim (its
 * top 4 significant bits, then the exact rest), four per rotated dim (16 significant bits); a
 * raw dim below 2^-13 of its 64-dim block's largest magnitude may lose bits below 2^-17 of that
 * magnitude. The 16-head kernel (short key sets) widens either way. */
#define CSKV_QK_FP4 0x100

CSKV_API int cskv_abi_version(void);
CSKV_API const char* cskv_strerror(int code);
CSKV_API const char* cskv_last_error(void);

/*
 * csa_compress / hca_compress - softmax-weighted pooling of m consecutive
 * tokens into one KV entry, then partial RoPE, then storage rounding.
 * (Page "DeepSeek-V4가 ... 달성하는 방법", section "두 가지 압축 전략: CSA 및
 * HCA": 4 tokens per CSA entry, 128 per HCA entry; page "딥시크 V4 분석 ...",
 * section "쉽게 이해하기": the pooling weights are learned per token.)
 *
 * For each sequence b and block j in [0, n_tok/m):
 *   a_i  = softmax_i(z[b, j*m + i]),  i = 0..m-1
 *   e    = sum_i a_i * x[b, j*m + i, :]
 *   (every step through the rotation below is evaluated in fp64 and the stored value is
 *   rounded once, from fp64, to its format)
 *   e    = e / sqrt(mean_d(e_d^2) + rms_eps)   if rms_eps > 0 (unit-gain RMSNorm
 *          of the entry: the pages' "KV normalisation", section "두 가지 압축
 *          전략: CSA 및 HCA"; rms_eps == 0 leaves e as pooled)
 *   e    = RoPE(e) on dims [D-d_rope, D) at p = pos0[b] + j*m + entry_pos_offset,
 *          pairs (2i, 2i+1) of that slice, theta_i = rope_base^(-2i/d_rope)
 *   out[b, out_entry0[b] + j, :] = bf16_rne(e)                       (CSKV_BF16)
 *     or  s = max|e| / 448 (1 if e == 0); codes = e4m3_rne_sat(e / s),
 *         out_scale[b, out_entry0[b] + j] = s                        (CSKV_FP8_E4M3)
 *     or  per 32 dims E = floor(log2 max|e_blk|) - 2 in [-127, 127] (-127 if all zero),
 *         codes = nearest e2m1 of e_blk / 2^E (ties to the even code, saturating at 6),
 *         out_scale = E + 127 as one byte per block                  (CSKV_MXFP4; OCP MX v1.0.
 *         The blog post on DeepSeek V4.1 Flash, jjy0501.blogspot.com, paragraph on the
 *         global attention state under "SWA Bounded Replay": the main KV cache is kept in
 *         HBM at FP4 precision.)
 *
 * x        [B, x_seq_stride] bf16; row r of sequence b at x + b*x_seq_stride + r*D
 *          (a ring slice works: rows are contiguous within a sequence)
 * z        [B, z_seq_stride] fp32 pooling logits, z + b*z_seq_stride + r
 * pos0     [B] int64, position of row 0 of each sequence
 * out      bf16 [B, out_seq_stride, D], fp8 codes [B, out_seq_stride, D] or MXFP4 codes
 *          [B, out_seq_stride, D/2]
 * out_scale fp32 [B, out_seq_stride] (fp8), uint8 E8M0 [B, out_seq_stride, D/32] (MXFP4);
 *          ignored for bf16
 * out_entry0 [B] int32 first entry slot written per sequence, or NULL (= 0)
 * Requirements: B >= 1, n_tok >= 0 and n_tok % m == 0, 1 <= m <= 1024,
 * D % 8 == 0 (MXFP4: D % 32 == 0) and 8 <= D <= 1024, d_rope % 8 == 0 and d_rope <= D,
 * x_seq_stride % 8 == 0, rms_eps finite and >= 0. hca_compress is the same
 * operation (named for its use with m = 128).
 */
CSKV_API int csa_compress(const uint16_t* x, int64_t x_seq_stride, const float* z, int64_t z_seq_stride,
                 const int64_t* pos0, int B, int n_tok, int D, int d_rope, int m,
                 int entry_pos_offset, float rope_base, int out_dtype, void* out, void* out_scale,
                 int64_t out_seq_stride, const int32_t* out_entry0, float rms_eps, void* stream);
CSKV_API int hca_compress(const uint16_t* x, int64_t x_seq_stride, const float* z, int64_t z_seq_stride,
                 const int64_t* pos0, int B, int n_tok, int D, int d_rope, int m,
                 int entry_pos_offset, float rope_base, int out_dtype, void* out, void* out_scale,
                 int64_t out_seq_stride, const int32_t* out_entry0, float rms_eps, void* stream);

/*
 * csa_index_key_pool - the indexer key of each compressed entry: the per-token
 * indexer keys of its m tokens pooled with the entry's softmax weights, then
 * stored in MXFP4 like the other indexer inputs.
 * (Page "DeepSeek-V4가 ... 달성하는 방법", section "두 가지 압축 전략: CSA 및
 * HCA": the FP4 indexer scores compressed entries; the pages give the entry keys
 * no source of their own, so this library derives them the way the entries are
 * derived: the same pooling weights, no RoPE.)
 *
 * For each sequence b and block j in [0, n_tok/m):
 *   a_i = softmax_i(z[b, j*m + i])                   (the weights of csa_compress)
 *   k   = sum_i a_i * xk[b, j*m + i, :]              (evaluated in fp64)
 *   per 32 values of k: E = floor(log2 max|block|) - 2, limited to [-3, 0]
 *     (an all-zero block takes -3); element code = nearest e2m1 magnitude of
 *     |v| / 2^E (ties to the even code, saturating at 6), sign bit 3 set for
 *     v < 0 (OCP MX v1.0 FP4)
 *   out_ik[b, out_entry0[b] + j, :]       = codes, element 2i in the low nibble of byte i
 *   out_ik_scale[b, out_entry0[b] + j, :] = E + 127 (E8M0)
 *
 * xk         [B, xk_seq_stride] bf16; row r of sequence b at xk + b*xk_seq_stride + r*D_I
 * z          [B, z_seq_stride] fp32 pooling logits (the ones given to csa_compress)
 * out_ik     [B, out_seq_stride, D_I/2] bytes; out_ik_scale [B, out_seq_stride, D_I/32]
 * out_entry0 [B] int32 first entry slot written per sequence, or NULL (= 0)
 * Requirements: B >= 1, n_tok % m == 0, 1 <= m <= 1024, D_I in {64, 128, 256,
 * 512}, xk 16-byte aligned, xk_seq_stride % 8 == 0 and >= n_tok*D_I.
 * Errors: CSKV_EINVAL (null, sizes, alignment), CSKV_ENOTSUP (D_I). The caller
 * owns every buffer; the call is asynchronous on `stream`.
 */
CSKV_API int csa_index_key_pool(const uint16_t* xk, int64_t xk_seq_stride, const float* z, int64_t z_seq_stride,
                       int B, int n_tok, int D_I, int m, uint8_t* out_ik, uint8_t* out_ik_scale,
                       int64_t out_seq_stride, const int32_t* out_entry0, void* stream);

/*
 * csa_index_topk - lightning-indexer scores and top-k selection.
 * (Page "DeepSeek-V4가 ... 달성하는 방법", section "두 가지 압축 전략: CSA 및
 * HCA": an FP4 indexer scores the compressed entries against the query and
 * the top-k, typically about 128, go on to attention. The score form is the
 * DSA lightning indexer's.)
 *
 *   s(b,t,j) = sum_h w[b,t,h] * max(0, sum_d q[b,t,h,d] * k[b,j,d]),  j < n_valid[b,t]
 * with q, k decoded from MXFP4. The scores are exact in fp32 as long as, per
 * score, the E8M0 exponent spread of the query plus that of the key plus that
 * of w stays within 2^24 / (H_I * D_I * 36) (8 for H_I*D_I = 1024). Entries
 * are ordered by (score descending, index ascending; -0 == +0) and the first
 * min(k, n_valid) are written; the rest of the row is -1 (score -inf).
 *
 * iq [B, T, H_I, D_I/2], iq_scale [B, T, H_I, D_I/32]
 * head_w [B, T, H_I] fp32, or NULL for all ones
 * ik [B, N_cap, D_I/2], ik_scale [B, N_cap, D_I/32]
 * n_valid [B, T] int32 in [0, N_cap]
 * out_idx [B, T, k] int32; out_score [B, T, k] fp32 or NULL
 * ws: device workspace of at least csa_index_topk_workspace_size(...) bytes
 * Requirements: D_I % 32 == 0, 32 <= D_I <= 512, 1 <= H_I <= 16, 1 <= k <= 1024.
 */
CSKV_API int csa_index_topk(const uint8_t* iq, const uint8_t* iq_scale, const float* head_w,
                   const uint8_t* ik, const uint8_t* ik_scale, const int32_t* n_valid, int B, int T,
                   int N_cap, int H_I, int D_I, int k, int32_t* out_idx, float* out_score, void* ws,
                   size_t ws_bytes, void* stream);
CSKV_API size_t csa_index_topk_workspace_size(int B, int T, int N_cap, int H_I, int D_I, int k);

/*
 * hybrid_attn_decode - T decode queries per sequence (T = 1: plain decode; T > 1:
 * a draft of T tokens checked in one step, causal inside the draft): shared-KV
 * MQA attention over compressed entries plus the sliding window, one joint
 * softmax per head. (Page "DeepSeek-V4가 ... 달성하는 방법", section "두 가지
 * 압축 전략: CSA 및 HCA": CSA attends to its top-k entries with a window branch
 * alongside, HCA attends to all of its entries; MQA shares one KV head; partial
 * RoPE. The blog post on DeepSeek V4.1 Flash (jjy0501.blogspot.com), section
 * "DSpark 추측 디코딩": the model checks
 * a block of drafted tokens at once.)
 *
 * Query r = b*T + j (sequence b, draft token j) at position t = q_pos[r]:
 *   keys = entries {topk_idx[r, i] >= 0} (CSA) or {0..n_entries[r]-1} (topk_idx == NULL, HCA)
 *          of sequence b, plus window tokens at positions [max(0, t-W+1), t], read raw
 *          from ring slot (position mod R) of sequence b and rotated at their own position
 *   q_rot = RoPE(q[r, h], t); logit = softmax_scale * g_h * q_rot . key, with
 *   g_h = 1 / sqrt(mean_d(q[r, h, d]^2) + q_rms_eps) if q_rms_eps > 0 (unit-gain
 *   RMSNorm of the query head, the pages' "query normalisation"), else 1
 *   out[r, h, :] = bf16_rne(sum softmax(logit) * key[:d_v]); out_lse[r, h] = ln(sum exp(logit))
 * Entries are stored rotated: bf16 [B, N_cap, D], fp8 codes [B, N_cap, D] with fp32
 * scales ckv_scale [B, N_cap] (value = code * scale), or MXFP4 codes [B, N_cap, D/2]
 * with E8M0 bytes ckv_scale [B, N_cap, D/32] (value = e2m1(code) * 2^(byte - 127)).
 *
 * q [B*T, H, D] bf16 (unrotated); q_pos [B*T] int64; n_entries [B*T] int32 <= N_cap
 * (causal inside a draft: each query its own count); topk_idx [B*T, k] int32 (each -1
 * or in [0, n_entries[r])) or NULL; win [B, R, D] bf16 rings of raw tokens (R = 0 means
 * R = W; a T-token step needs R >= W + T - 1 so that no query's window has been
 * overwritten); out [B*T, H, d_v] bf16; out_lse [B*T, H] fp32 or NULL; ws of at least
 * hybrid_attn_decode_workspace_size(B*T, ...) bytes (none when that size is 0): the partial
 * results of the key splits, merged by a second launch. Calls sharing a workspace must not run
 * concurrently. A key set needing more than 64 splits of 4096 keys is refused (CSKV_ENOTSUP).
 * Requirements: D % 32 == 0, D <= 1024, d_v % 16 == 0, d_v <= D, d_v <= 512,
 * d_rope % 8 == 0, d_rope <= min(D, 64), 1 <= H <= 128, W >= 0, T >= 1, R >= W + T - 1 when
 * W > 0 (CSKV_EINVAL otherwise; with R = 0 a draft of T > 1 tokens is refused),
 * W + k or W + N_cap fits int32, q_rms_eps finite and >= 0.
 */
CSKV_API int hybrid_attn_decode(const uint16_t* q, const int64_t* q_pos, const void* ckv,
                       const void* ckv_scale, int ckv_dtype, int N_cap, const int32_t* n_entries,
                       const int32_t* topk_idx, int k, const uint16_t* win, int W, int B, int H,
                       int D, int d_rope, int d_v, float rope_base, float softmax_scale,
                       uint16_t* out, float* out_lse, void* ws, size_t ws_bytes, float q_rms_eps,
                       int T, int R, void* stream);
CSKV_API size_t hybrid_attn_decode_workspace_size(int B, int H, int d_v, int N_cap, int k, int W, int dense);

/*
 * hybrid_attn_decode_append - the decode state update of a layer and its attention in one call:
 * the same result as cskv_ring_append(x_new, z_new, pos, ring_x, ring_z, B, T, D, R) with
 * pos[b] = q_pos[b*T], followed by hybrid_attn_decode(..., win = ring_x, ...) on the same
 * stream. (Page "딥시크 V4 분석 ...", section "쉽게 이해하기": every layer keeps the latest 128
 * tokens raw beside its compressed entries; each decode step adds its token to that window and
 * attends over it.) The attention takes the step's new tokens from x_new and writes them to
 * their ring slots in the same launch, one workgroup per sequence (no reader of the call needs
 * those slots: R >= W + T - 1). Where a block of m tokens completes at this step, the caller
 * runs cskv_ring_append, the compression and then hybrid_attn_decode instead, since the
 * compression reads the new token from the ring.
 *
 * Arguments as in hybrid_attn_decode, with win replaced by ring_x [B, R, D] bf16 (written:
 * slots (q_pos[b*T] + i) mod R, i < T), and x_new [B, T, D] bf16 (16-byte aligned), z_new
 * [B, T] fp32 pooling logits or NULL, ring_z [B, R] fp32 (written with z_new). Queries of a
 * sequence must sit at consecutive positions: q_pos[b*T + j] = q_pos[b*T] + j. Workspace:
 * hybrid_attn_decode_workspace_size(B*T, ...). Requirements as in hybrid_attn_decode, and
 * R >= T, B * R < 2^30, ring_x and x_new non-NULL (CSKV_EINVAL otherwise).
 */
CSKV_API int hybrid_attn_decode_append(const uint16_t* q, const int64_t* q_pos, const void* ckv,
                       const void* ckv_scale, int ckv_dtype, int N_cap, const int32_t* n_entries,
                       const int32_t* topk_idx, int k, uint16_t* ring_x, float* ring_z,
                       const uint16_t* x_new, const float* z_new, int W, int B, int H, int D,
                       int d_rope, int d_v, float rope_base, float softmax_scale, uint16_t* out,
                       float* out_lse, void* ws, size_t ws_bytes, float q_rms_eps, int T, int R,
                       void* stream);

/*
 * cskv_attn_path - which attention kernel hybrid_attn_decode, _noalloc and _prefill run (and
 * their *_workspace_size functions plan for): 0 (the default) chooses by the call's shape, the
 * 16-head kernel for short key sets of few queries (at most 512 keys per query and at most 4096
 * (query, key) pairs in the call) and the 64-head kernel otherwise; 1 forces the 64-head kernel,
 * 2 the 16-head kernel.
 * Both compute the same attention (parity-tested each); the choice moves only time and
 * workspace size. A process-wide setting, read at each call: set it before sizing a workspace
 * and keep it until the calls that use that workspace have been issued; not for concurrent use
 * from several host threads. Errors: CSKV_EINVAL (path outside [0, 2]).
 */
CSKV_API int cskv_attn_path(int path);

/*
 * cskv_attn_cu_budget - the number of compute units the 64-head kernel's key-split plan counts
 * on (hybrid_attn_decode, _noalloc, _prefill and their *_workspace_size functions). The plan
 * weighs each workgroup's fixed prologue and epilogue against the rounds of workgroups the CUs
 * take; 0 (the default) counts the whole GPU (256 CUs). A caller that runs other kernels beside
 * the attention calls on another stream passes the share it expects them to leave, so that the
 * plan takes fewer, longer splits. Results are the same for every budget (the split count only
 * reorders the fp32 sums of a head's partials); time and workspace size change. Process-wide,
 * with the same rules as cskv_attn_path (set before sizing a workspace, keep while the calls
 * using it are issued, not for concurrent use from several host threads).
 * Errors: CSKV_EINVAL (cus outside [0, 4096]).
 */
CSKV_API int cskv_attn_cu_budget(int cus);

/*
 * hybrid_attn_decode_noalloc - hybrid_attn_decode without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It computes the same result with the same kernels; the
 * key-split partials live in a static device array of CSKV_NOALLOC_SCRATCH_BYTES that each GPU
 * holds from the first call on it until the process ends. No call allocates or frees device
 * memory.
 *
 * Arguments, layouts and requirements as in hybrid_attn_decode. A call whose
 * hybrid_attn_decode_workspace_size(B*T, ...) exceeds CSKV_NOALLOC_SCRATCH_BYTES is refused
 * with CSKV_EWORKSPACE before anything is enqueued. All calls on one GPU share that GPU's
 * array (every partial is written before it is read, so nothing needs clearing between calls):
 * calls that may overlap on one GPU (different streams, or host threads) race and must not
 * be issued.
 */
#define CSKV_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
CSKV_API int hybrid_attn_decode_noalloc(const uint16_t* q, const int64_t* q_pos, const void* ckv,
                       const void* ckv_scale, int ckv_dtype, int N_cap, const int32_t* n_entries,
                       const int32_t* topk_idx, int k, const uint16_t* win, int W, int B, int H,
                       int D, int d_rope, int d_v, float rope_base, float softmax_scale,
                       uint16_t* out, float* out_lse, float q_rms_eps, int T, int R, void* stream);

/*
 * hybrid_attn_prefill - the same attention for every row of one prompt. (Page
 * "DeepSeek-V4가 ... 달성하는 방법", section "두 가지 압축 전략: CSA 및 HCA", as for
 * hybrid_attn_decode: every prompt position is a query of CSA's top-k entries plus its
 * window, or of all HCA entries; causally it sees only entries of blocks already complete
 * and tokens up to itself.)
 * Row r is position t = pos0 + r. It sees entries j < min(N, floor((t+1)/m))
 * (CSA: those listed in topk_idx[r]; HCA: all of them when topk_idx == NULL)
 * and the raw tokens x at positions [max(pos0, t-W+1), t], rotated at their
 * own positions.
 *
 * q [T, H, D] bf16; ckv / ckv_scale as in decode with N entries;
 * topk_idx [T, k] or NULL; x [T, D] bf16 raw tokens of the prompt;
 * out [T, H, d_v] bf16; out_lse [T, H] fp32 or NULL; ws as in decode.
 * Requirements as in decode, plus m >= 1.
 */
CSKV_API int hybrid_attn_prefill(const uint16_t* q, int64_t pos0, int T, const void* ckv,
                        const void* ckv_scale, int ckv_dtype, int N, const int32_t* topk_idx,
                        int k, const uint16_t* x, int W, int H, int D, int d_rope, int d_v, int m,
                        float rope_base, float softmax_scale, uint16_t* out, float* out_lse,
                        void* ws, size_t ws_bytes, float q_rms_eps, void* stream);
CSKV_API size_t hybrid_attn_prefill_workspace_size(int T, int H, int d_v, int N, int k, int W, int dense);

/*
 * cskv_ring_append - decode state update: write each sequence's T new raw
 * tokens and pooling logits into its ring at slots (pos[b] + i) mod R. (The
 * window keeps the latest W tokens: page "딥시크 V4 분석 ...", section "쉽게
 * 이해하기"; a ring of R >= W + T - 1 slots keeps every window of a T-token
 * step intact while its later tokens are appended.)
 *
 * x_new [B, T, D] bf16; z_new [B, T] fp32 or NULL; pos [B] int64 (position of token 0);
 * ring_x [B, R, D] bf16; ring_z [B, R] fp32 or NULL (with z_new).
 * Requirements: D % 8 == 0, 1 <= T <= R.
 */
CSKV_API int cskv_ring_append(const uint16_t* x_new, const float* z_new, const int64_t* pos,
                     uint16_t* ring_x, float* ring_z, int B, int T, int D, int R, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSKV_H_ */
