/*
 * fa.h -- exact attention (FlashAttention forward) and paged-KV decode for AMD
 * Instinct MI355X (gfx950), C ABI.
 *
 * What is computed (pages: "Phase 08 -- Inference Optimization at Depth",
 * Concepts list and Lab 01; screna.ai interview notes, FlashAttention,
 * online-softmax and MHA/MQA/GQA blocks):
 *
 *   S = scale * Q K^T,  causal: S[i][j] = -inf for j > i,
 *   O = softmax(S) V,   L[i] = ln sum_j exp(S[i][j])   (natural log, fp32)
 *
 * computed tile by tile with the online-softmax recurrence (running row max and
 * row sum, output accumulator rescaled per key tile), so the N x N score matrix
 * is never stored: only O and L are written.  Query head h reads K/V head
 * h / (Hq / Hkv) (grouped-query heads; Hkv == 1 is multi-query).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers to memory the caller allocated.
 *     Tensors are dense, contiguous, row-major, with the layouts stated below,
 *     and every tensor pointer must be 16-byte aligned.
 *   - Inputs are read-only.  o and lse are fully overwritten and must not alias
 *     any input.  The library never allocates, frees or synchronises.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).  Work
 *     is enqueued on it and the call returns; errors inside a running kernel are
 *     not reported by the call.  Setting the environment variable FA_DEBUG=1
 *     makes every call synchronise the stream and report kernel errors.
 *   - Arguments are validated on the host before any HIP call; a failed check
 *     returns its status code and launches nothing.
 *   - Every size is at least 1: B, Hq, Hkv, N, num_seqs, chunk, max_pages_per_seq
 *     and num_pages below 1 return FA_ERR_SHAPE.  So do sizes past the kernels'
 *     limits: a launch must stay below 2^31 work-items, and the bf16 kernels
 *     address one (batch, head) slice of N x d values through a 32-bit byte
 *     range, so N * d * 2 must not exceed 2^32 - 1 (N < 2^24 at d = 128).
 *   - Validation order: sizes (FA_ERR_SHAPE), head dimension / page size
 *     (FA_ERR_UNSUPPORTED), scale (FA_ERR_SCALE), pointers (FA_ERR_NULL, then
 *     FA_ERR_ALIGN), workspace (FA_ERR_WORKSPACE).
 *   - Thread safety: the library has no mutable global state besides a
 *     thread-local copy of the last HIP error text and, for
 *     fa_decode_paged_noalloc, its per-GPU device scratch and the cached device
 *     addresses of that scratch (looked up under a lock).
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FA_OK              0 /* enqueued (or nothing to do)                        */
#define FA_ERR_NULL        1 /* a required pointer is NULL                         */
#define FA_ERR_SHAPE       2 /* a size < 1, Hq % Hkv != 0, or past a kernel limit */
#define FA_ERR_UNSUPPORTED 3 /* head dim not 64/128, page_size not 16             */
#define FA_ERR_SCALE       4 /* scale is NaN or infinite                           */
#define FA_ERR_ALIGN       5 /* a tensor pointer is not 16-byte aligned            */
#define FA_ERR_WORKSPACE   6 /* decode workspace NULL or smaller than required     */
#define FA_ERR_HIP         7 /* a HIP launch / runtime call failed                 */
#define FA_ERR_SCRATCH     8 /* sizes exceed the fixed scratch of a _noalloc call  */

/*
 * fa_fwd -- bf16 exact-attention forward (prefill).
 *
 * Pages: "Phase 08", Concepts (online softmax; FlashAttention tiling: Q in
 * blocks of B_r rows, K/V streamed in blocks of B_c columns; only O and the
 * logsumexp L stored; causal tiles that span the diagonal are handled apart
 * from full and fully-masked ones) and Lab 01 steps 2 and 4 (tile Q, iterate
 * K/V blocks, online softmax; skip future tiles entirely); getnybble
 * "Inference Optimization -- Advanced", question 5 (parallelism over query
 * blocks); screna.ai MHA/MQA/GQA block (grouped K/V heads).
 *
 *   q   [B, Hq,  N, d] bf16      k, v [B, Hkv, N, d] bf16
 *   o   [B, Hq,  N, d] bf16 (out, fp32 accumulation, rounded to nearest even)
 *   lse [B, Hq,  N]    fp32 (out, natural-log logsumexp of the scaled scores)
 *   d in {64, 128}; Hq % Hkv == 0; B, N >= 1 and N * d * 2 < 2^32; causal: 0 or
 *   1 (query i sees keys j <= i); scale: any finite float (usually 1/sqrt(d)).
 * Returns FA_OK or a status code above.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           void* stream);

/*
 * fa_fwd_splitk_workspace_size -- bytes of device workspace fa_fwd_splitk needs
 * for these sizes: 0 when the launch has at least 256 (query block of 256 rows,
 * head) items and nothing is split, else the fp32 partials (O and logsumexp) of
 * the blocks whose key range is cut into chunks.  Returns 0 when an argument is
 * out of range.
 */
size_t fa_fwd_splitk_workspace_size(int B, int Hq, int N, int d, int causal);

/*
 * fa_fwd_splitk -- fa_fwd for launches with few heads (one GPU's share of a
 * head-sharded model, short batches): the same operation, tensors, outputs and
 * status codes, with the key range of each query block cut into chunks when the
 * launch has fewer than 256 (query block, head) items, so the chunks spread over
 * all the compute units instead of the heaviest causal block setting the time.
 *
 * Pages: as fa_fwd; the chunks' partial (O, logsumexp) are combined by the
 * log-sum-exp merge of the split-K decode ("Phase 08", Lab 03 step 4: split-K
 * over the keys), which gives the same exact attention.
 *
 *   workspace: device memory of at least fa_fwd_splitk_workspace_size(B, Hq, N,
 *   d, causal) bytes, 16-byte aligned, owned by the caller (may be NULL when that
 *   size is 0); contents on entry do not matter.  Calls sharing a workspace must
 *   be ordered (same stream).
 * Returns FA_OK or a status code above (FA_ERR_WORKSPACE for a missing or short
 * workspace).
 */
int fa_fwd_splitk(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_f32 -- the same operation in fp32 throughout (inputs, the P V product
 * with unrounded fp32 probabilities, accumulation and O).  Same pages, same
 * parameter list and layouts as fa_fwd with every tensor fp32.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               void* stream);

/*
 * fa_fwd_ex -- fa_fwd with a sliding window and/or an ALiBi bias (bf16).
 *
 * Pages: "Phase 08", Lab 01 extensions row (sliding-window attention as in
 * Mistral; ALiBi bias support).  Same tensors, layouts, outputs and status codes
 * as fa_fwd, plus:
 *   window        >= 0.  W > 0 keeps, for query i, only keys j >= i - W + 1 (the
 *                 last W positions up to and including i); requires causal = 1
 *                 (FA_ERR_UNSUPPORTED otherwise).  0: no window.
 *   alibi_slopes  device pointer to Hq fp32 slopes m_h, or NULL for no bias; the
 *                 score of (i, j) for query head h becomes
 *                 scale * q_i . k_j - m_h * |i - j| (before masking), and lse is the
 *                 logsumexp of these biased scores.  4-byte aligned.
 * With window = 0 and alibi_slopes = NULL it computes exactly what fa_fwd does.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
              int window, const float* alibi_slopes, void* stream);

/*
 * fa_prefill_paged -- chunked prefill: a chunk of `chunk` new query tokens per
 * sequence attends to the sequence's paged KV cache, causal within the chunk.
 *
 * Pages: "Phase 08", Concepts (chunked prefill splits a long prompt into pieces;
 * paged attention) and Lab 03 steps 1 and 4 (16-token pages behind an
 * indirection table).  Sequence s holds ctx_lens[s] cached tokens whose last
 * `chunk` are the chunk's own (their K/V already written to the cache); chunk row
 * r is the token at position ctx_lens[s] - chunk + r and sees every cached token
 * at a position <= its own.
 *
 *   q          [S, Hq, chunk, d] bf16         o   [S, Hq, chunk, d] bf16 (out)
 *   lse        [S, Hq, chunk] fp32 (out, natural-log logsumexp)
 *   kpages, vpages, page_table, num_pages, max_pages_per_seq: as fa_decode_paged.
 *   ctx_lens   [S] int32, chunk <= ctx_lens[s] <= max_pages_per_seq * page_size
 *              (device data).  Cache slots at or beyond ctx_lens[s] never affect
 *              the result, whatever they hold.  A value outside that range, or a
 *              page id outside [0, num_pages), gives wrong output but no access
 *              outside the buffers: the kernel clamps ctx_lens[s] into
 *              [chunk, max_pages_per_seq * page_size] and page ids into
 *              [0, num_pages - 1].
 *   d in {64, 128}; page_size == 16; Hq % Hkv == 0; 1 <= chunk <=
 *   max_pages_per_seq * page_size; any finite scale.  No workspace.
 */
int fa_prefill_paged(const void* q, const void* kpages, const void* vpages,
                     const int32_t* page_table, const int32_t* ctx_lens,
                     void* o, float* lse, int num_seqs, int Hq, int Hkv, int d,
                     int chunk, int page_size, int max_pages_per_seq,
                     int num_pages, float scale, void* stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs for these
 * sizes: D = rowsum(dO * O) and L * log2(e) per row (fp32), plus fp32 partial
 * sums of dK and dV when a K/V head's query heads are split over several
 * workgroups (few K/V heads).  Returns 0 when an argument is out of range.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d);

/*
 * fa_bwd -- bf16 exact-attention backward: the gradients of a loss with respect
 * to q, k and v, given its gradient dout with respect to the forward's output.
 *
 * Pages: "Phase 08", Concepts (the FlashAttention backward keeps only O and the
 * logsumexp L from the forward, not the N x N matrix) and Lab 01 step 6 (the
 * optional backward).  The probabilities are recomputed tile by tile from q, k
 * and lse; with S = scale * q k^T (masked as in fa_fwd), P = exp(S - L),
 * D = rowsum(dout * o), dP = dout v^T and dS = P * (dP - D):
 *   dq = scale * dS k,   dk = scale * dS^T q,   dv = P^T dout,
 * dk and dv summed over the query heads that share a K/V head.
 *
 *   q, o, dout, dq [B, Hq, N, d] bf16;   k, v, dk, dv [B, Hkv, N, d] bf16
 *   lse [B, Hq, N] fp32: the logsumexp fa_fwd returned for the same q, k, v,
 *       causal and scale; o its output.
 *   dq, dk, dv are written completely (out, fp32 accumulation rounded to
 *   nearest even); they must not alias the inputs.
 *   workspace: device memory of at least fa_bwd_workspace_size(B, Hq, Hkv, N, d)
 *   bytes, 16-byte aligned, owned by the caller; contents on entry do not matter.
 *   Calls sharing a workspace must be ordered (same stream).
 *   d in {64, 128}; Hq % Hkv == 0; B, N >= 1, N * d * 2 < 2^32; causal 0 or 1;
 *   any finite scale.
 * Returns FA_OK or a status code above (FA_ERR_WORKSPACE for a missing or short
 * workspace).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_paged_workspace_size -- bytes of device workspace fa_decode_paged
 * needs for these sizes (fp32 split partials and their logsumexps).  Returns 0
 * when an argument is out of range (negative size, unsupported d / page_size).
 */
size_t fa_decode_paged_workspace_size(int num_seqs, int Hq, int d,
                                      int max_pages_per_seq, int page_size);

/*
 * fa_decode_paged -- one-query-per-sequence attention over a paged KV cache
 * (decode), split along the context and merged with a log-sum-exp combine.
 *
 * Pages: "Phase 08", Concepts (KV cache; paged attention: the cache lives in
 * non-contiguous fixed-size pages) and Lab 03 steps 1 and 4 (16-token pages; a
 * kernel that reaches non-contiguous pages through an indirection table).
 * Each split's partial result is combined with the online-softmax rescaling
 * algebra of the Lab 01 talking points applied to whole splits.
 *
 *   q          [S, Hq, d] bf16          (S = num_seqs, one query per sequence)
 *   kpages     [num_pages, Hkv, page_size, d] bf16   (one (page, head) block is
 *   vpages     [num_pages, Hkv, page_size, d] bf16    page_size*d contiguous)
 *   page_table [S, max_pages_per_seq] int32: logical page p of sequence s is
 *              physical page page_table[s][p]; only entries p < ceil(ctx/page)
 *              are read.
 *   ctx_lens   [S] int32: tokens in each sequence's cache, 0 <= ctx_lens[s] <=
 *              max_pages_per_seq * page_size.  Cache slots at or beyond
 *              ctx_lens[s] are never allowed to affect the result, whatever they
 *              hold (NaN included).  ctx_lens[s] == 0 gives O = 0, L = -inf.
 *   o          [S, Hq, d] bf16 (out);  lse [S, Hq] fp32 (out, natural log).
 *   d in {64, 128}; page_size == 16; Hq % Hkv == 0.
 *   workspace: device memory of at least
 *   fa_decode_paged_workspace_size(num_seqs, Hq, d, max_pages_per_seq,
 *   page_size) bytes, owned by the caller, 16-byte aligned; its contents on
 *   entry do not matter.  Two calls that share a workspace must be ordered
 *   (same stream).
 * num_pages: physical pages in each pool (>= 1).  Device-side values out of
 * range give wrong output but no access outside the buffers: the kernels clamp
 * ctx_lens[s] into [0, max_pages_per_seq * page_size] and page ids into
 * [0, num_pages - 1].
 */
int fa_decode_paged(const void* q, const void* kpages, const void* vpages,
                    const int32_t* page_table, const int32_t* ctx_lens,
                    void* o, float* lse,
                    int num_seqs, int Hq, int Hkv, int d, int page_size,
                    int max_pages_per_seq, int num_pages, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_paged_noalloc -- fa_decode_paged without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * Same operation, arguments, layouts and status codes as fa_decode_paged, minus
 * workspace / workspace_bytes.  The split partials go to a device scratch array
 * the library holds, one copy per GPU, of fa_decode_paged_noalloc_max_scratch()
 * bytes (32 MiB), kept until the process ends.  Sizes whose workspace
 * (fa_decode_paged_workspace_size) exceeds it return FA_ERR_SCRATCH and launch
 * nothing.  The call itself allocates nothing: the scratch's device address is
 * looked up once per device, on the first call that uses it.  Every call on a
 * GPU shares that GPU's scratch: calls that overlap on one GPU (different streams,
 * or different host threads without ordering) race and give wrong output; calls
 * ordered on one stream are fine.
 */
int fa_decode_paged_noalloc(const void* q, const void* kpages, const void* vpages,
                            const int32_t* page_table, const int32_t* ctx_lens,
                            void* o, float* lse,
                            int num_seqs, int Hq, int Hkv, int d, int page_size,
                            int max_pages_per_seq, int num_pages, float scale,
                            void* stream);

/* Bytes of the device scratch behind fa_decode_paged_noalloc (per GPU). */
size_t fa_decode_paged_noalloc_max_scratch(void);

/*
 * fa_decode_paged_int8 -- fa_decode_paged over an INT8 KV cache with group-wise
 * scales (half the cache bytes of bf16, plus the scales).
 *
 * Pages: screna.ai KV-cache quantization block (an 8-bit cache halves the KV
 * memory; group-wise scales keep the accuracy of per-tensor ones or better) and
 * "Phase 08", Lab 03 step 4 (paged attention).  The cached value of channel c of
 * token t is kpages[pg][h][t][c] * kscale[pg][h][t][c / group] (V alike).
 *
 *   kpages, vpages  [num_pages, Hkv, page_size, d] int8, 16-byte aligned
 *   kscale, vscale  [num_pages, Hkv, page_size, d / group] fp32, 4-byte aligned
 *   group           32 (channels per scale); other values FA_ERR_UNSUPPORTED
 *   everything else (q, o, lse, page_table, ctx_lens, workspace and its size from
 *   fa_decode_paged_workspace_size, status codes) as fa_decode_paged.  Slots at or
 *   beyond ctx_lens[s] never affect the result, whatever values or scales they hold.
 */
int fa_decode_paged_int8(const void* q, const int8_t* kpages, const float* kscale,
                         const int8_t* vpages, const float* vscale,
                         const int32_t* page_table, const int32_t* ctx_lens,
                         void* o, float* lse, int num_seqs, int Hq, int Hkv, int d,
                         int page_size, int group, int max_pages_per_seq,
                         int num_pages, float scale, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * fa_status_string -- static text for a status code.  For FA_ERR_HIP it is the
 * text of the last HIP error seen by the calling thread.
 */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
