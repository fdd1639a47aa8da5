/*
 * fa.h — C ABI of the exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention as one fused, tiled
 * pass per query tile: score tiles Q·Kᵀ, the softmax and the product with V
 * never leave the compute unit, the running row max m and normaliser l of the
 * online softmax rescale the partial output, and only O and the per-row
 * logsumexp reach device memory.  Sources of the definition:
 *   - "Flash Attention 是什么：2026 最新原理、架构演进与实战详解" (ai.lansai.wang):
 *     技术原理 › 核心工作机制 (standard flow S = Q·Kᵀ, softmax, ·V; tiling;
 *     online softmax; recomputation from the saved max and sum);
 *     关键术语解析 §4 (the m and l update equations); 常见误解澄清, 误解一
 *     (the result is exact; only rounding order differs).
 *   - lqnn.cn "为什么Flash突然成了AI圈的高频词" §2.1 (Q/K/V as [B, H, N, d],
 *     e.g. [1, 32, 16384, 128]) and §3.3 (causal flag; softmax scale with
 *     default 1/sqrt(d_k)).
 *   - 0539edu.com "Flash不是那个被时代淘汰的插件" §2 (a KV page pool reserved
 *     at load time, fixed 256-token pages handed to sequences; decode is
 *     memory-bound, prefill compute-bound).
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major and contiguous, innermost dimension last.
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     never allocates, frees or keeps a pointer after returning.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; the library never synchronises.
 *   - Arguments are validated on the host BEFORE anything is launched; on a
 *     validation error nothing is enqueued and the output buffers are left
 *     untouched.  A failed launch returns FA_ERR_HIP.
 *   - Contents of device-resident index arrays (block tables, lengths) cannot
 *     be checked without a synchronisation and are trusted: out-of-range
 *     values are undefined behaviour.
 *   - Calls on one stream are ordered; calls that share output or workspace
 *     buffers on different streams race.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_PTR = 1,     /* a required pointer is NULL                              */
  FA_ERR_BAD_SHAPE = 2,    /* a size is negative/zero where it may not be, or overflows */
  FA_ERR_UNSUPPORTED = 3,  /* head dim, dtype or page size this build does not handle  */
  FA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than *_workspace_bytes()       */
  FA_ERR_HIP = 5,          /* the HIP runtime reported an error (no device, launch)    */
  FA_ERR_SCRATCH_TOO_SMALL = 6  /* the library's static scratch cannot hold the problem  */
} fa_status;

typedef enum {
  FA_F32 = 0,              /* IEEE fp32 in and out, fp32 arithmetic                     */
  FA_BF16 = 1              /* bf16 in and out, bf16 matrix products accumulated in fp32 */
} fa_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_str(fa_status s);

/* Text of the last HIP runtime error seen by this thread's calls into the
 * library (static string, never NULL; "no error" if none). */
const char* fa_last_hip_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fa_version(void);

/*
 * fa_forward — O = softmax(scale · Q Kᵀ [+ causal mask]) V and the row logsumexp.
 *
 *   dt      FA_BF16 (head dim 64 or 128) or FA_F32 (head dim 64 or 128).
 *   B,H,N,d batch, heads, sequence length (queries = keys = N), head dim.
 *           B, H >= 1; N >= 0 (N == 0 is a no-op returning FA_OK).
 *   q,k,v   [B, H, N, d] of dtype dt.
 *   o       [B, H, N, d] of dtype dt (written).  bf16 outputs are rounded to
 *           nearest-even from the fp32 result.
 *   lse     [B, H, N] fp32 (written) or NULL to skip: the natural log of the
 *           sum over visible keys of exp(scale · q_i·k_j).  It is the only
 *           statistic a recomputing backward needs.
 *   causal  non-zero: query i sees keys 0..i (future keys masked).
 *   scale   softmax scale, finite and > 0 (else FA_ERR_BAD_SHAPE); callers
 *           wanting the usual default pass 1/sqrt(d).
 *           Must be finite.
 * Work: 4·d·pairs·B·H flops, pairs = N(N+1)/2 causal, N² otherwise; extra
 * device memory: none (no N×N buffer).
 */
fa_status fa_forward(fa_dtype dt, int B, int H, int N, int d,
                     const void* q, const void* k, const void* v,
                     void* o, float* lse, int causal, float scale, void* stream);

/*
 * Workspace the backward needs, in bytes: two fp32 per query row (the row
 * dot product D_i = dO_i · O_i, and the row's logsumexp in base-2 units), each
 * array rounded up to 256 bytes.  O(B·H·N); no N×N.
 */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_backward — gradients of L = Σ O∘dO through the forward above, with the
 * attention probabilities recomputed tile by tile from Q, K and the saved
 * logsumexp instead of being stored (the explainer's recomputation).
 *
 *   dt            FA_BF16 only; head dim 64 or 128.
 *   q,k,v         forward inputs [B, H, N, d] bf16.
 *   o, dout       forward output and its gradient [B, H, N, d] bf16.
 *   lse           [B, H, N] fp32 as written by fa_forward on the same inputs.
 *   dq,dk,dv      [B, H, N, d] bf16 (written), fp32-accumulated, rounded
 *                 to nearest-even.
 *   workspace     device buffer of >= fa_backward_workspace_bytes() bytes,
 *                 owned by the caller; contents on entry are ignored.
 *   causal, scale as in fa_forward.
 * Deterministic: every output element is accumulated in a fixed order.
 */
fa_status fa_backward(fa_dtype dt, int B, int H, int N, int d,
                      const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes,
                      int causal, float scale, void* stream);

/*
 * fa_forward_gqa — fa_forward with grouped key/value heads (GQA; MQA when
 * Hkv == 1): Explainer 进阶学习路径 §4 names the multi-query / grouped-query
 * adaptation.  q, o: [B, H, N, d]; k, v: [B, Hkv, N, d]; query head h attends
 * with key/value head h / (H / Hkv).  H must be a multiple of Hkv.  Other
 * arguments, LSE layout and errors as fa_forward.
 */
fa_status fa_forward_gqa(fa_dtype dt, int B, int H, int Hkv, int N, int d,
                         const void* q, const void* k, const void* v,
                         void* o, float* lse, int causal, float scale, void* stream);

/*
 * fa_forward_varlen — a batch of sequences of different lengths packed
 * without padding (Explainer 使用门槛和条件 §4: per-sample lengths with no
 * padding waste).
 *   cu_seqlens  [B+1] int32 on the device: sequence b owns packed rows
 *               cu_seqlens[b] .. cu_seqlens[b+1]-1; cu_seqlens[0] = 0,
 *               non-decreasing, cu_seqlens[B] = total.  The table is not
 *               validated; the kernels clamp each bound to [0, total] and
 *               each length to max_seqlen, so a malformed table never makes
 *               them touch memory outside the buffers, but rows it leaves
 *               uncovered are not written.
 *   max_seqlen  the largest length (host value; sizes the launch).  It must
 *               be >= every sequence's length: rows of a longer sequence past
 *               max_seqlen are not computed (nor written), and the rows of
 *               that sequence that are written get NaN in O and the LSE, so
 *               the error shows in the outputs (the table lives on the device
 *               and is not read on the host).
 *   q, o        [total, H, d];  k, v  [total, Hkv, d] (token-major, heads
 *               interleaved per token).
 *   lse         [H, total] fp32 or NULL.
 * Attention (and the causal mask) stays inside each sequence.  dt FA_BF16 or
 * FA_F32; other arguments and errors as fa_forward_gqa.
 */
fa_status fa_forward_varlen(fa_dtype dt, int B, int H, int Hkv, int max_seqlen, int total, int d,
                            const int32_t* cu_seqlens, const void* q, const void* k, const void* v,
                            void* o, float* lse, int causal, float scale, void* stream);

/* Backward of fa_forward_gqa: dk, dv are [B, Hkv, N, d] and sum the
 * gradients of every query head of the group.  Workspace as fa_backward. */
fa_status fa_backward_gqa(fa_dtype dt, int B, int H, int Hkv, int N, int d,
                          const void* q, const void* k, const void* v,
                          const void* o, const void* dout, const float* lse,
                          void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes,
                          int causal, float scale, void* stream);

/* Workspace of fa_backward_varlen in bytes: one fp32 per (head, packed row). */
size_t fa_backward_varlen_workspace_bytes(int H, int total, int d);

/* Backward of fa_forward_varlen (packed layouts as there; lse [H, total]).
 * As there, max_seqlen must cover every sequence: a longer sequence gets NaN
 * gradients in the rows that are written and none past max_seqlen. */
fa_status fa_backward_varlen(fa_dtype dt, int B, int H, int Hkv, int max_seqlen, int total, int d,
                             const int32_t* cu_seqlens, const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes,
                             int causal, float scale, void* stream);

/*
 * Workspace for fa_decode_paged in bytes: per (sequence, head, KV split) a
 * partial running max, normaliser and unnormalised output row in fp32; a
 * split is half a 256-token page, so at most 2·max_blocks_per_seq splits
 * per sequence.
 */
size_t fa_decode_workspace_bytes(int num_seqs, int H, int d, int max_blocks_per_seq);

/*
 * fa_decode_paged — one new query token per sequence against that sequence's
 * paged KV cache (split over pages, then merged exactly through the running
 * max / normaliser algebra of the online softmax).
 *
 *   num_seqs,H,d        sequences (>= 1), heads (>= 1), head dim (128 or 64).
 *   page_size           tokens per page; this build supports 256.
 *   num_pages           pages in the pool (>= 1).
 *   max_blocks_per_seq  columns of block_table (>= 1).
 *   q                   [num_seqs, H, d] bf16.
 *   kv_pool             [num_pages, 2, page_size, H, d] bf16; index 0 of the
 *                       second dim holds K, index 1 holds V.
 *   block_table         [num_seqs, max_blocks_per_seq] int32 (device): entry
 *                       b of row s is the physical page holding tokens
 *                       b·page_size .. b·page_size+page_size-1 of sequence s.
 *                       Entries past ceil(L_s/page_size) are never read.
 *   seq_lens            [num_seqs] int32 (device), 1 <= L_s <=
 *                       max_blocks_per_seq·page_size.  Slots >= L_s in the
 *                       last page are never read.
 * Device-side contents are not validated, but they never make the kernels
 * touch memory outside the buffers: a table entry outside [0, num_pages) is
 * clamped into the pool (a wrong page is read), lengths past
 * max_blocks_per_seq·page_size are cut there, and L_s <= 0 yields O = 0 and
 * LSE = -inf for that sequence.
 *   o                   [num_seqs, H, d] bf16 (written).
 *   lse                 [num_seqs, H] fp32 (written) or NULL.
 *   scale               softmax scale, finite and > 0.
 *   workspace           >= fa_decode_workspace_bytes() bytes, caller-owned.
 * The query sees all L_s cached keys (no causal mask).  Deterministic.
 */
fa_status fa_decode_paged(int num_seqs, int H, int d, int page_size,
                          int num_pages, int max_blocks_per_seq,
                          const void* q, const void* kv_pool,
                          const int32_t* block_table, const int32_t* seq_lens,
                          void* o, float* lse, float scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_paged_gqa — fa_decode_paged with grouped key/value heads (GQA;
 * MQA when Hkv == 1): "Flash Attention 是什么" (ai.lansai.wang) 进阶学习路径 §4
 * names the multi-query / grouped-query adaptation.
 *   q        [num_seqs, H, d] bf16; query head h reads key/value head
 *            h / (H / Hkv).  H must be a multiple of Hkv.
 *   kv_pool  [num_pages, 2, page_size, Hkv, d] bf16.
 * Each K/V row of the pool is read once for all H / Hkv query heads that
 * share it.  Workspace: fa_decode_workspace_bytes(num_seqs, H, d,
 * max_blocks_per_seq) suffices.  Other arguments, outputs and errors as
 * fa_decode_paged; with Hkv == H it is fa_decode_paged.
 */
fa_status fa_decode_paged_gqa(int num_seqs, int H, int Hkv, int d, int page_size,
                              int num_pages, int max_blocks_per_seq,
                              const void* q, const void* kv_pool,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* o, float* lse, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_paged_gqa_static — fa_decode_paged_gqa for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument and no allocation
 * of any kind.  The decode partials go to a static device array of
 * fa_decode_static_scratch_bytes() bytes (16 MiB) that the library holds on
 * every GPU it runs on until the process ends; its address is looked up once
 * per device, on the first call made with that device current.
 *   Arguments, outputs and results as fa_decode_paged_gqa (Hkv == H is the
 *   plain paged decode).  A problem whose partials, fa_decode_workspace_bytes(
 *   num_seqs, H, d, max_blocks_per_seq), exceed the scratch returns
 *   FA_ERR_SCRATCH_TOO_SMALL before anything is launched.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap
 *   on one GPU (different streams, or different host threads without
 *   ordering) race and corrupt each other's results.  Nothing in the scratch
 *   needs to start at zero (every partial that is read is written first in
 *   the same call).
 */
size_t fa_decode_static_scratch_bytes(void);
fa_status fa_decode_paged_gqa_static(int num_seqs, int H, int Hkv, int d, int page_size,
                                     int num_pages, int max_blocks_per_seq,
                                     const void* q, const void* kv_pool,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     void* o, float* lse, float scale, void* stream);

/*
 * fa_prefill_paged — chunked prefill over a paged KV cache: every sequence
 * appends a chunk of new tokens to a cached prefix, the chunk's K/V already
 * written to the pool, and its queries attend through the block table.  The
 * pool of 256-token pages is the decode one (0539edu.com "Flash不是那个被时代
 * 淘汰的插件" §2); reusing a cached prefix instead of recomputing it is the
 * prefix caching of zwxr.cn §5.2.
 *   cu_seqlens_q  [B+1] int32 (device): sequence b's queries are packed rows
 *                 cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q.
 *   max_seqlen_q  largest chunk (host value; sizes the launch); a longer
 *                 chunk is handled as fa_forward_varlen handles a sequence
 *                 longer than max_seqlen (NaN in its written rows).
 *   q, o          [total_q, H, d] bf16; lse [H, total_q] fp32 or NULL.
 *   kv_pool       [num_pages, 2, 256, Hkv, d] bf16; query head h reads
 *                 key/value head h / (H / Hkv).
 *   block_table   [B, max_blocks_per_seq] int32 (device), max_blocks_per_seq
 *                 <= 512 (else FA_ERR_UNSUPPORTED).
 *   seq_lens_k    [B] int32 (device): cached keys of sequence b, prefix plus
 *                 chunk.  The chunk's queries are the last positions: with
 *                 causal, query i of a chunk of n sees keys 0 .. i + L_b - n
 *                 (a query that sees none gets O = 0, LSE = -inf); without,
 *                 every query sees all L_b keys.
 * Device-side contents are not validated but never make the kernel touch
 * memory outside the buffers (table entries are clamped into the pool,
 * lengths into max_blocks_per_seq·256 and [0, total_q]).  d 64 or 128; bf16
 * only; other errors as fa_forward.
 */
fa_status fa_prefill_paged(int B, int H, int Hkv, int d, int max_seqlen_q, int total_q,
                           const int32_t* cu_seqlens_q, const void* q,
                           const void* kv_pool, int page_size, int num_pages,
                           const int32_t* block_table, int max_blocks_per_seq,
                           const int32_t* seq_lens_k, void* o, float* lse,
                           int causal, float scale,
                           const float* rope_cos, const float* rope_sin,
                           int rope_rows, int rope_interleaved, void* stream);

/*
 * fa_forward_rope — the forward with the rotary position embedding applied
 * to Q and K inside the kernel, from precomputed cosine / sine tables (the
 * fused RoPE with a lookup table of 0539edu.com "Flash不是那个被时代淘汰的
 * 插件" §3; the rotated Q/K are never written to memory).
 *   cu_seqlens  NULL: dense, q/o [B, H, N, d] and k/v [B, Hkv, N, d];
 *               else packed as fa_forward_varlen (N = max_seqlen, total rows).
 *   rope_cos, rope_sin  fp32 [rope_rows, d/2], 16-byte aligned; rope_rows
 *               >= N.  A row at position p (its index in its sequence) has
 *               feature pair i rotated by the angle whose cosine / sine are
 *               rope_cos[p][i], rope_sin[p][i]:
 *               (x, y) -> (x·cos − y·sin, x·sin + y·cos).
 *   rope_interleaved  0: pair i = features (i, i + d/2); 1: (2i, 2i+1).
 * The rotation runs in fp32 on the bf16 inputs and is rounded to bf16 (RNE)
 * before the products.  bf16 only.  Other arguments and errors as
 * fa_forward_gqa / fa_forward_varlen.
 *
 * fa_prefill_paged takes the same four rotary arguments (NULL tables: none)
 * and rotates its queries only, at positions i + L_b − n: the cached keys are
 * expected to be stored already rotated.
 */
fa_status fa_forward_rope(fa_dtype dt, int B, int H, int Hkv, int N, int total, int d,
                          const int32_t* cu_seqlens, const void* q, const void* k,
                          const void* v, void* o, float* lse, int causal, float scale,
                          const float* rope_cos, const float* rope_sin, int rope_rows,
                          int rope_interleaved, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
