/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa.so).
 *
 * Three calls, one per part of the method:
 *
 *   fa_fwd     O = softmax(scale * Q K^T) V with the per-row log-sum-exp, by IO-aware
 *              tiles and an online softmax (running max m, running sum l, rescaled fp32
 *              accumulator, one division by l at the end).
 *              Pages: V2/V3 article (aiqz.cc), sections "IO瓶颈分析", "V2算法优化" and
 *              "Warp级并行"; interview answer "flash attention呢" (agentalpha.top),
 *              标准答 part 1; study card airsota.com/?p=1562, sections 三 and 四 ①.
 *   fa_bwd     dQ, dK, dV from dO, recomputing the local scores from Q, K and the saved
 *              log-sum-exp instead of storing P.
 *              Pages: interview answer 标准答 part 2 (recompute); study card section
 *              四 ②; self-test page "二十四：Flash Attention自测题", section D (the dV,
 *              dP, dS, dQ, dK relations).
 *   fa_decode  one new token per sequence over a variable-length KV cache: the cache
 *              is cut into chunks attended independently (partial O and LSE), then the
 *              partials are merged by the online-softmax update.
 *              Pages: interview answer, 高频追问 2; self-test page, section F.
 *
 * Further variants:
 *
 *   fa_fwd_varlen    the forward over a packed batch of variable-length sequences
 *                    (prefix offsets instead of padding).
 *                    Pages: self-test page, section C (padding masks and variable-length
 *                    sequences).
 *   fa_fwd_dropout / fa_bwd_dropout  the forward and backward with dropout on P, the
 *                    mask regenerated from a counter-based generator (Philox4x32-10).
 *                    Pages: self-test page, section C.
 *   fa_quantize_fp8  two-pass E4M3 block quantisation of Q or K (step = block max / 448).
 *   fa_fwd_fp8       the forward with Q K^T on the E4M3 matrix cores (fp32 accumulation).
 *                    Pages: V2/V3 article, section FP8低精度 and its formula block.
 *   fa_decode_paged  the split-KV decode over a KV cache kept in fixed-size pages named
 *                    by a per-sequence block table, read page by page where it lies.
 *                    Pages: self-test page, section F (why paged attention or a decode
 *                    kernel is still needed); interview answer, 高频追问 2 (blocked decode
 *                    reading the paged KV blocks directly).
 *   fa_decode_noalloc  fa_decode with its partials in a static per-device array, for
 *                    callers that cannot allocate device memory.
 *
 * Conventions shared by every call
 * --------------------------------
 *  * Tensors are [batch, heads, seq, dim] (self-test page section A; the article's
 *    Python demo), addressed by element strides for the batch, head and sequence
 *    dimensions; the dim dimension is contiguous (stride 1).  Strides and base
 *    pointers must keep every row 16-byte aligned.
 *  * MHA / GQA / MQA: Hq query heads, Hkv key/value heads, Hq % Hkv == 0; query head
 *    h reads KV head h / (Hq / Hkv) (self-test page section F).
 *  * scale multiplies Q K^T before the softmax; callers normally pass 1/sqrt(D)
 *    (self-test page section C; study card section 二).  It must be > 0 and finite.
 *  * causal: key j is visible to query i iff j <= i + (Lk - Nq), Lk being the number
 *    of valid keys of that batch entry (lower-triangular for Nq == Lk; the last query
 *    sees the whole cache).
 *  * Variable-length KV: keys at positions >= Lk do not exist.  Their memory is never
 *    read into a result (it may hold NaN).  A query row with no visible key gets
 *    O = 0 and LSE = -inf, and zero gradients.
 *  * LSE is natural-log, in the units of the scaled scores: LSE_i = m_i + ln(l_i).
 *  * Non-finite inputs (self-test page, section G: locating NaN outputs): in fa_fwd,
 *    fa_fwd_varlen and fa_decode, a NaN in query row i makes O_i and LSE_i NaN, and a
 *    NaN in a key row j makes O and LSE NaN for exactly the query rows that see j;
 *    every other row is computed as if the NaN were absent.  A NaN in a value row
 *    reaches the O rows that see it and may reach rows of the same 64-key block that
 *    do not (their weight 0 times NaN); LSE never depends on V.  The backward makes no
 *    such promise: non-finite values spread through the gradient sums.
 *  * Every pointer named "device" is device memory owned by the caller; the library
 *    never allocates, frees or synchronises, keeps no mutable global state (apart from
 *    fa_decode_noalloc's static per-device array, described there) and is safe to call
 *    from several host threads.  Work is enqueued asynchronously on the
 *    caller's HIP stream (`stream` is a hipStream_t; NULL means the null stream);
 *    outputs are valid once that stream reaches the enqueued work.
 *  * Validation runs on the host before anything is enqueued: a non-FA_OK return
 *    means nothing was launched and no output was touched.  FA_ERR_LAUNCH reports a
 *    launch failure from the HIP runtime.  No C++ exception crosses this ABI.
 *  * Device code is built for gfx950 only; fa_device_supported() says whether a
 *    device can run it.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_PTR = 1,    /* a required pointer is NULL                         */
  FA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent              */
  FA_ERR_DTYPE = 3,       /* unknown or unsupported dtype combination            */
  FA_ERR_STRIDE = 4,      /* a stride or pointer breaks the 16-byte alignment    */
  FA_ERR_UNSUPPORTED = 5, /* valid request this build does not implement (e.g. D) */
  FA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the query says       */
  FA_ERR_DEVICE = 7,      /* no current HIP device, or it is not gfx950          */
  FA_ERR_LAUNCH = 8,      /* the HIP runtime rejected a kernel launch            */
  FA_ERR_ARG = 9          /* scale not finite and > 0, or another bad scalar     */
} fa_status;

typedef enum fa_dtype {
  FA_BF16 = 0,
  FA_F32 = 1
} fa_dtype;

/* ---------------------------------------------------------------------------------
 * Forward.
 *   q  [B, Hq,  Nq, D]  in_dtype  (device)
 *   k  [B, Hkv, Nk, D]  in_dtype  (device)
 *   v  [B, Hkv, Nk, D]  in_dtype  (device)
 *   o  [B, Hq,  Nq, D]  out_dtype (device, written)
 *   lse  contiguous [B, Hq, Nq] fp32 (device, written), or NULL if not wanted
 *   kv_lens  [B] int32 (device), valid keys per batch entry (clamped to [0, Nk]), or
 *            NULL meaning Nk for every entry
 *   k and v may be NULL when Nk == 0 (nothing is read).
 * Supported: in_dtype FA_BF16 with D in {64, 128} and out_dtype FA_BF16 or FA_F32;
 *            in_dtype FA_F32 with D = 64 and out_dtype FA_F32.
 * Sizes: B, Hq, Hkv >= 1; Nq, Nk >= 0 (Nq == 0 launches nothing).  Nk == 0 or an
 *        all-zero kv_lens gives O = 0, LSE = -inf.
 * ------------------------------------------------------------------------------- */
typedef struct fa_fwd_args {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *kv_lens;
  int64_t q_stride[3]; /* elements: batch, head, seq */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int32_t B, Hq, Hkv, Nq, Nk, D;
  int32_t in_dtype;  /* fa_dtype */
  int32_t out_dtype; /* fa_dtype */
  float scale;
  int32_t causal;    /* 0 or 1 */
} fa_fwd_args;

fa_status fa_fwd(const fa_fwd_args *args, void *stream);

/* ---------------------------------------------------------------------------------
 * Backward (bf16, D in {64, 128}).
 *   q, k, v, o, dout  as in the forward (o is the forward output, dout = dL/dO), bf16
 *   lse   contiguous [B, Hq, Nq] fp32, natural log, as written by fa_fwd (device)
 *   dq    [B, Hq,  Nq, D] bf16 (device, written)
 *   dk    [B, Hkv, Nk, D] bf16 (device, written; GQA: summed over the group's query
 *         heads in fp32 before rounding)
 *   dv    [B, Hkv, Nk, D] bf16 (device, written)
 *   kv_lens, scale, causal as in the forward; rows of dk/dv at positions >= Lk are 0.
 * The workspace (device, caller-owned, at least fa_bwd_workspace_bytes() bytes, 16-byte
 * aligned, any contents) holds two fp32 planes [B, Hq, Nq], each padded to a multiple of
 * 256 bytes: LSE * log2 e, then -D_i = -rowsum(dO * O); it is written by the call
 * itself.  Two kernels run in stream order: dQ (one workgroup per query tile,
 * recomputing S and dP; it also forms and stores the row statistics) and dK/dV (one
 * workgroup per key tile).  No atomics are used: results are bitwise reproducible run
 * to run.
 * ------------------------------------------------------------------------------- */
typedef struct fa_bwd_args {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  const int32_t *kv_lens;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int64_t do_stride[3];
  int64_t dq_stride[3];
  int64_t dk_stride[3];
  int64_t dv_stride[3];
  int32_t B, Hq, Hkv, Nq, Nk, D;
  int32_t dtype; /* FA_BF16 */
  float scale;
  int32_t causal;
} fa_bwd_args;

/* Bytes of workspace fa_bwd needs for these sizes (0 if the sizes are invalid). */
size_t fa_bwd_workspace_bytes(const fa_bwd_args *args);
fa_status fa_bwd(const fa_bwd_args *args, void *workspace, size_t workspace_bytes,
                 void *stream);

/* ---------------------------------------------------------------------------------
 * Split-KV decode (bf16 cache, D in {64, 128}).
 *   q        [Bs, Hq, D] bf16 (device), one new token per sequence
 *   k_cache  [Bs, Hkv, cache_len, D] bf16 (device)
 *   v_cache  [Bs, Hkv, cache_len, D] bf16 (device)
 *   seq_lens [Bs] int32 (device): valid cached keys of each sequence; values are
 *            clamped to [0, max_len] on the device
 *   o        [Bs, Hq, D] out_dtype (device, written)
 *   lse      contiguous [Bs, Hq] fp32 (device, written) or NULL
 *   max_len  host-side bound on seq_lens, 0 <= max_len <= cache_len; sizes the grid
 *            so no device-to-host copy is needed
 *   split_len keys per chunk, a positive multiple of 128; chunk c of sequence s covers
 *            keys [c*split_len, min((c+1)*split_len, L_s)).
 * The workspace (device, at least fa_decode_workspace_bytes() bytes) receives each
 * chunk's partial output and LSE, [Bs, Hq, ceil(max_len/split_len)] x (D + 1) fp32;
 * a second kernel merges them:
 *   M = max_c LSE_c, w_c = exp(LSE_c - M), O = sum_c w_c O_c / sum_c w_c,
 *   LSE = M + ln(sum_c w_c).
 * A sequence with L_s = 0 gets O = 0, LSE = -inf.
 * ------------------------------------------------------------------------------- */
typedef struct fa_decode_args {
  const void *q;
  const void *k_cache, *v_cache;
  const int32_t *seq_lens;
  void *o;
  float *lse;
  int64_t q_stride[2]; /* elements: sequence, head */
  int64_t k_stride[3]; /* elements: sequence, head, position */
  int64_t v_stride[3];
  int64_t o_stride[2];
  int32_t Bs, Hq, Hkv, D;
  int32_t cache_len;
  int32_t max_len;
  int32_t split_len;
  int32_t in_dtype;  /* FA_BF16 */
  int32_t out_dtype; /* FA_BF16 or FA_F32 */
  float scale;
} fa_decode_args;

size_t fa_decode_workspace_bytes(const fa_decode_args *args);
fa_status fa_decode(const fa_decode_args *args, void *workspace, size_t workspace_bytes,
                    void *stream);

/* ---------------------------------------------------------------------------------
 * Decode that allocates nothing: fa_decode with its workspace taken from a static
 * device array of FA_DECODE_NOALLOC_MAX_WORKSPACE_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends.
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The call itself allocates and frees
 * nothing (no hipMalloc, hipFree or allocating library routine); the caller passes the
 * inputs and outputs exactly as for fa_decode.
 *   args  as for fa_decode.
 * Returns FA_ERR_WORKSPACE, launching nothing, when fa_decode_workspace_bytes(args)
 * exceeds FA_DECODE_NOALLOC_MAX_WORKSPACE_BYTES (32 MiB: e.g. 64 sequences x 32 query
 * heads x 16 chunks at D = 128 need 16.9 MB), and FA_ERR_DEVICE when no device is
 * current.  The first call on a device looks up that device's array address (once per
 * device, with the device current) and keeps it.
 * Every call on one GPU shares that GPU's array, which keeps the previous call's
 * partials; nothing in it needs clearing, since the merge reads only partials the same
 * call's split kernel wrote.  Calls that overlap on one GPU (other streams, other host
 * threads) race on the array: the caller must order them.
 * ------------------------------------------------------------------------------- */
#define FA_DECODE_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)32 << 20)
fa_status fa_decode_noalloc(const fa_decode_args *args, void *stream);

/* ---------------------------------------------------------------------------------
 * Forward and backward with dropout on P (bf16, D in {64, 128}).
 * Pages: self-test page, section C (how dropout is done without storing the mask).
 *   args, workspace: as fa_fwd / fa_bwd
 *   p_drop  dropout probability in [0, 1), taken in steps of 1/256: t = round(256 p);
 *           t == 0 runs the plain call
 *   seed    64-bit key of the mask generator
 * Element (b, h, i, j) is kept iff byte 4a + e of Philox4x32-10(counter = (2 (j / 32) +
 * (j / 4) % 2, i, h, b), key = (seed low, seed high)) is >= t, with a = (j / 8) % 4,
 * e = j % 4 and byte n at bits 8 (n % 4) of word n / 4; kept probabilities are scaled
 * by 256 / (256 - t).  O = (P * mask * scale) V; LSE is that of the undropped scores.
 * The backward regenerates the same mask (pass the forward's p_drop and seed):
 * dV = (P * mask * scale)^T dO, dP = (dO V^T) * mask * scale, D_i = rowsum(dO * O).
 * FA_ERR_ARG for p_drop outside [0, 1); FA_ERR_UNSUPPORTED for fp32 inputs.
 * ------------------------------------------------------------------------------- */
fa_status fa_fwd_dropout(const fa_fwd_args *args, float p_drop, uint64_t seed, void *stream);
fa_status fa_bwd_dropout(const fa_bwd_args *args, float p_drop, uint64_t seed, void *workspace,
                         size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Forward over a packed batch of B variable-length sequences (bf16, D in {64, 128}).
 *   q  [total_q, Hq,  D] bf16 (device); rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1
 *      are the queries of sequence b
 *   k  [total_k, Hkv, D] bf16 (device); rows cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1
 *      are the keys of sequence b; v likewise
 *   cu_seqlens_q, cu_seqlens_k  [B + 1] int32 (device): non-decreasing row offsets with
 *      [0] = 0 and [B] = total; on the device each is clamped into [previous, total],
 *      so no read or write leaves the packed tensors whatever they hold
 *   max_seqlen_q  host-side bound on every sequence's query count (sizes the grid);
 *      rows of a longer sequence past it are not written
 *   o  [total_q, Hq, D] out_dtype (device, written); lse contiguous [Hq, total_q] fp32
 *      (device, written) or NULL
 *   strides: elements between consecutive rows ([0]) and heads ([1]); dim stride 1.
 * Each sequence attends its own keys only; causal alignment, GQA, scale and LSE follow
 * the forward.  A sequence with no keys gets O = 0, LSE = -inf.  k and v may be NULL
 * when total_k == 0.  Supported: in_dtype FA_BF16, out_dtype FA_BF16 or FA_F32.
 * ------------------------------------------------------------------------------- */
typedef struct fa_fwd_varlen_args {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *cu_seqlens_q, *cu_seqlens_k;
  int64_t q_stride[2]; /* elements: row, head */
  int64_t k_stride[2];
  int64_t v_stride[2];
  int64_t o_stride[2];
  int32_t B, Hq, Hkv, D;
  int32_t total_q, total_k;
  int32_t max_seqlen_q;
  int32_t in_dtype;  /* FA_BF16 */
  int32_t out_dtype; /* FA_BF16 or FA_F32 */
  float scale;
  int32_t causal;
} fa_fwd_varlen_args;

fa_status fa_fwd_varlen(const fa_fwd_varlen_args *args, void *stream);

/* ---------------------------------------------------------------------------------
 * Split-KV decode over a paged KV cache (bf16, D in {64, 128}).
 *   k_pages, v_pages  page pools of num_pages pages (device), addressed by element
 *      strides k_stride = {page, head, row within the page}; dim stride 1.  Both
 *      [num_pages, Hkv, page_size, D] and [num_pages, page_size, Hkv, D] fit.
 *   block_table  int32 (device), row s at block_table + s * table_stride: entry j names
 *      the page holding positions j*page_size .. (j+1)*page_size - 1 of sequence s.
 *      Entries at or past ceil(L_s / page_size) are never read; an entry outside
 *      [0, num_pages) reads its page as zeros (no memory outside the pools is touched).
 *   page_size  a power of two, 16 .. 2^20
 *   max_pages_per_seq  usable entries per table row: max_len <= max_pages_per_seq *
 *      page_size, table_stride >= max_pages_per_seq
 *   split_len  as in fa_decode, at most 4096
 *   q, seq_lens, o, lse, max_len, dtypes and scale as in fa_decode.
 * Workspace: fa_decode_paged_workspace_bytes() bytes of chunk partials, merged as in
 * fa_decode.  A sequence with L_s = 0 gets O = 0, LSE = -inf.
 * ------------------------------------------------------------------------------- */
typedef struct fa_decode_paged_args {
  const void *q;
  const void *k_pages, *v_pages;
  const int32_t *block_table;
  const int32_t *seq_lens;
  void *o;
  float *lse;
  int64_t q_stride[2]; /* elements: sequence, head */
  int64_t k_stride[3]; /* elements: page, head, row within the page */
  int64_t v_stride[3];
  int64_t o_stride[2];
  int64_t table_stride; /* elements between block_table rows */
  int32_t Bs, Hq, Hkv, D;
  int32_t num_pages, page_size, max_pages_per_seq;
  int32_t max_len;
  int32_t split_len;
  int32_t in_dtype;  /* FA_BF16 */
  int32_t out_dtype; /* FA_BF16 or FA_F32 */
  float scale;
} fa_decode_paged_args;

size_t fa_decode_paged_workspace_bytes(const fa_decode_paged_args *args);
fa_status fa_decode_paged(const fa_decode_paged_args *args, void *workspace,
                          size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * E4M3 block quantisation (D = 128, block = 64).
 *   x       [B, H, N, D] bf16 (device), strides in elements
 *   codes   [B, H, N, D] uint8 (device, written): OCP E4M3 codes of x / Delta, rounded
 *           to nearest even; strides in bytes
 *   scales  contiguous [B, H, ceil(N / 64)] fp32 (device, written): Delta of each block of
 *           64 rows, max|x| / 448 (one fp32 division), 1 for an all-zero block
 * ------------------------------------------------------------------------------- */
typedef struct fa_quantize_fp8_args {
  const void *x;
  void *codes;
  float *scales;
  int64_t x_stride[3];     /* elements: batch, head, row */
  int64_t codes_stride[3]; /* bytes: batch, head, row */
  int32_t B, H, N, D;
  int32_t block;           /* 64 */
} fa_quantize_fp8_args;

fa_status fa_quantize_fp8(const fa_quantize_fp8_args *args, void *stream);

/* ---------------------------------------------------------------------------------
 * Forward with E4M3 Q and K (D = 128).
 *   q  [B, Hq, Nq, D] E4M3 codes with q_scales contiguous [B, Hq, ceil(Nq / 64)] fp32
 *   k  [B, Hkv, Nk, D] E4M3 codes with k_scales contiguous [B, Hkv, ceil(Nk / 64)] fp32
 *      (as written by fa_quantize_fp8; code strides in bytes)
 *   v  [B, Hkv, Nk, D] bf16; o, lse, kv_lens, scale, causal as in fa_fwd
 * S = scale * (Delta_q q_hat)(Delta_k k_hat)^T is formed on the E4M3 matrix cores with
 * fp32 accumulation; the softmax, P (bf16) V and the outputs are those of fa_fwd.
 * out_dtype FA_BF16 or FA_F32.
 * ------------------------------------------------------------------------------- */
typedef struct fa_fwd_fp8_args {
  const void *q, *k, *v;
  const float *q_scales, *k_scales;
  void *o;
  float *lse;
  const int32_t *kv_lens;
  int64_t q_stride[3]; /* bytes: batch, head, seq */
  int64_t k_stride[3]; /* bytes */
  int64_t v_stride[3]; /* elements */
  int64_t o_stride[3]; /* elements */
  int32_t B, Hq, Hkv, Nq, Nk, D;
  int32_t block;       /* 64 */
  int32_t out_dtype;   /* FA_BF16 or FA_F32 */
  float scale;
  int32_t causal;
} fa_fwd_fp8_args;

fa_status fa_fwd_fp8(const fa_fwd_fp8_args *args, void *stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char *fa_status_str(int status);

/* 1 if HIP device `device` is a gfx950 part this library was built for, else 0.
 * Makes HIP runtime calls. */
int fa_device_supported(int device);

/* Library ABI version: (major << 16) | minor. */
int fa_version(void);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* FA_H_ */
