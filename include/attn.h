/*
 * attn.h -- exact attention forward on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn.so.  Three operations:
 *
 *   attn_prefill       exact scaled-dot-product attention over whole
 *                      sequences (optionally causal, grouped-query heads),
 *                      computed the FlashAttention way: Q/K/V tiles are
 *                      staged on chip, QK^T and PV run on the matrix cores,
 *                      a running row max and row sum rescale the partial
 *                      output tile by tile, and the N x N score matrix never
 *                      reaches device memory.
 *                      ("推理加速" interview notes, section FlashAttention:
 *                      tiling, on-chip block attention, online softmax, only
 *                      the final output written back, mathematically equal to
 *                      standard attention; chenyy20.com "抱infra脚", section
 *                      Flash Attention 基本原理 / 核心技术: tiling, online
 *                      softmax and kernel fusion of QK + softmax + PV.)
 *
 *   attn_prefill_paged the same over a paged KV cache, for a chunk of new
 *                      query tokens at the end of each cached sequence
 *                      (chunked prefill).
 *
 *   attn_decode_paged  one new query token per sequence against a paged KV
 *                      cache, Flash-Decoding style: the cached keys of each
 *                      sequence are cut into chunks processed in parallel,
 *                      each producing a partial output and its log-sum-exp,
 *                      and a second small kernel merges the partials with the
 *                      online-softmax formula, accumulating in fp32.
 *                      ("GPU Kernel 调度：大模型推理的拐点 2026", paragraphs on
 *                      Flash Decoding and its reduce-kernel cost; chenyy20.com
 *                      "抱infra脚", section Paged Attention: fixed-size cache
 *                      blocks mapped through a block table.)
 *
 * Conventions shared by both operations
 * -------------------------------------
 *  - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *    allocates nothing, keeps no state between calls and may be called from
 *    several host threads at once.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without waiting.  Outputs are valid once the stream has
 *    reached that point.
 *  - Tensors are contiguous, row-major, head_dim innermost.  bf16 is the
 *    IEEE-style bfloat16 (1-8-7) bit pattern in a uint16.
 *  - Query head h uses key/value head h / (n_q_heads / n_kv_heads)
 *    (consecutive query heads share a KV head).
 *  - Causal visibility is bottom-right aligned: key j is visible to query i
 *    iff j <= i + (seqlen_k - seqlen_q).  A query row with no visible key
 *    gets O = 0 and lse = -inf.
 *  - lse is the natural-log log-sum-exp of the visible scaled scores
 *    (scale * q.k), in fp32.
 *  - Internally: scores, softmax statistics and output accumulators are
 *    fp32; for bf16 inputs the probabilities are rounded to bf16 (nearest
 *    even) as the PV matrix-core operand and O is rounded to bf16 (nearest
 *    even) once at the end.  The fp32 path never rounds below fp32.
 *  - Errors are returned as attn_status_t; nothing is thrown across the ABI.
 *    All argument checks run on the host before any HIP call: on a non-OK
 *    status nothing has been enqueued and no output has been touched, except
 *    ATTN_ERR_LAUNCH (the launch itself failed; outputs are undefined).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                      */
    ATTN_ERR_ALIGN = 2,       /* a tensor pointer is not 16-byte aligned          */
    ATTN_ERR_SHAPE = 3,       /* negative size, heads not a multiple, bad sizes   */
    ATTN_ERR_DTYPE = 4,       /* unknown dtype code                               */
    ATTN_ERR_UNSUPPORTED = 5, /* valid but not implemented (head_dim, block_size,
                                 dtype for this operation, num_splits range)      */
    ATTN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required       */
    ATTN_ERR_LAUNCH = 7       /* the HIP launch reported an error                 */
} attn_status_t;

typedef enum {
    ATTN_BF16 = 0,            /* bf16 inputs and output                           */
    ATTN_F32 = 1              /* fp32 inputs and output                           */
} attn_dtype_t;

typedef void *attn_stream_t;  /* a hipStream_t */

/* Largest num_splits accepted by attn_decode_paged. */
#define ATTN_MAX_SPLITS 256

/*
 * attn_prefill -- O = softmax(scale * Q K^T [+ causal mask]) V per (batch, head).
 *
 *   q    [batch, seqlen_q, n_q_heads,  head_dim]   dtype
 *   k    [batch, seqlen_k, n_kv_heads, head_dim]   dtype
 *   v    [batch, seqlen_k, n_kv_heads, head_dim]   dtype
 *   o    [batch, seqlen_q, n_q_heads,  head_dim]   dtype, written
 *   lse  [batch, n_q_heads, seqlen_q]              fp32, written; may be NULL
 *
 * Supported: dtype ATTN_BF16 or ATTN_F32; head_dim 64 or 128.
 * batch == 0 or seqlen_q == 0 is a no-op (pointers may then be NULL);
 * seqlen_k == 0 gives O = 0, lse = -inf.  q, k, v, o must be 16-byte
 * aligned, lse 4-byte aligned.  q/k/v must not overlap o/lse.
 * Returns ATTN_ERR_SHAPE for negative sizes, non-positive head counts,
 * n_q_heads % n_kv_heads != 0, or element counts above 2^31 per tensor;
 * ATTN_ERR_UNSUPPORTED for another head_dim; ATTN_ERR_DTYPE for an unknown
 * dtype code.
 */
attn_status_t attn_prefill(const void *q, const void *k, const void *v,
                           void *o, float *lse,
                           int batch, int seqlen_q, int seqlen_k,
                           int n_q_heads, int n_kv_heads, int head_dim,
                           int causal, float scale, attn_dtype_t dtype,
                           attn_stream_t stream);

/*
 * attn_prefill_paged -- exact attention of a chunk of new query tokens over
 * keys and values held in a paged cache: the prefill of one chunk of a long
 * prompt whose earlier chunks (and this chunk's own keys and values) are
 * already cached.  ("抱infra脚", sections Chunked Prefill and Paged
 * Attention: a long prompt is processed a chunk at a time against the cache,
 * whose fixed-size blocks are reached through a block table; "推理加速"
 * interview notes, section FlashAttention, for the computation itself.)
 *
 *   q            [batch, seqlen_q, n_q_heads, head_dim]             bf16
 *   k_cache      [num_blocks, block_size, n_kv_heads, head_dim]     bf16
 *   v_cache      [num_blocks, block_size, n_kv_heads, head_dim]     bf16
 *   block_table  [batch, max_blocks_per_seq] int32 (as attn_decode_paged)
 *   ctx_lens     [batch] int32: cached keys of each sequence, including the
 *                seqlen_q keys of this chunk, which are its last ones
 *   o            [batch, seqlen_q, n_q_heads, head_dim] bf16, written
 *   lse          [batch, n_q_heads, seqlen_q] fp32, written; may be NULL
 *
 * Query i of sequence b is the token at position ctx_lens[b] - seqlen_q + i,
 * so with causal != 0 it sees keys j <= i + ctx_lens[b] - seqlen_q (the
 * bottom-right alignment of attn_prefill with seqlen_k = ctx_lens[b]); a row
 * with no visible key gets O = 0, lse = -inf.  Without causal every cached
 * key is visible.  Cache slots past ctx_lens[b] are never read.
 *
 * Supported: bf16, head_dim 64 or 128, block_size 16.  Device-side contract
 * violations do not fault: a sequence whose ctx_lens entry is negative or
 * exceeds max_blocks_per_seq * block_size, or whose needed block ids fall
 * outside [0, num_blocks), gets NaN in o and lse.  Host-side checks and
 * status codes are those of attn_decode_paged (no workspace).
 */
attn_status_t attn_prefill_paged(const void *q, const void *k_cache, const void *v_cache,
                                 const int32_t *block_table, const int32_t *ctx_lens,
                                 void *o, float *lse,
                                 int batch, int seqlen_q, int n_q_heads, int n_kv_heads, int head_dim,
                                 int num_blocks, int block_size, int max_blocks_per_seq,
                                 int causal, float scale, attn_stream_t stream);

/*
 * attn_decode_num_splits -- the number of key chunks per sequence that
 * attn_decode_paged will use for these arguments.  num_splits >= 1 is
 * returned unchanged (after the range check of attn_decode_paged);
 * num_splits <= 0 asks for the library's choice, which depends only on the
 * arguments given here (never on device data): one chunk when the table
 * holds fewer than 1024 tokens per sequence (the Flash-Decoding threshold of
 * "GPU Kernel 调度：大模型推理的拐点 2026", advice 2: below it splitting is
 * slower), else chunks of about 2048 tokens of the longest sequence the
 * table can hold, or more chunks (none shorter than 256 tokens) when that is
 * needed for about 256 (chunk, sequence, KV head) items, one per compute
 * unit, to occupy the GPU.  Two chunks of a table of at most 2048 tokens
 * become one (no merge); a count that at most doubles into two items of
 * four KV heads per compute unit is doubled.  Returns 0 for invalid
 * arguments.
 */
int attn_decode_num_splits(int batch, int n_kv_heads, int max_blocks_per_seq,
                           int block_size, int num_splits);

/*
 * attn_decode_workspace_bytes -- size of the scratch buffer attn_decode_paged
 * needs for these arguments.  It holds what Flash-Decoding keeps between its
 * two kernels ("GPU Kernel 调度：大模型推理的拐点 2026", paragraphs on Flash
 * Decoding and its cost: each chunk's partial output with its log-sum-exp,
 * kept in fp32 because fp16 partials lose accuracy as the chunk count
 * grows): the per-chunk partial outputs
 * [batch, n_q_heads, splits, head_dim] fp32 followed by their log-sum-exps
 * [batch, n_q_heads, splits] fp32 (splits = attn_decode_num_splits(...)),
 * then 256 bytes of scheduling state (a work counter, set by each call
 * itself, so its contents on entry do not matter either).  Returns 0 for
 * invalid arguments.
 */
size_t attn_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                   int max_blocks_per_seq, int block_size, int num_splits);

/*
 * attn_decode_paged -- one query token per sequence over a paged KV cache.
 *
 *   q            [batch, n_q_heads, head_dim]                       bf16
 *   k_cache      [num_blocks, block_size, n_kv_heads, head_dim]     bf16
 *   v_cache      [num_blocks, block_size, n_kv_heads, head_dim]     bf16
 *   block_table  [batch, max_blocks_per_seq] int32: physical block of each
 *                logical block; entries past a sequence's last block are
 *                ignored (conventionally -1)
 *   ctx_lens     [batch] int32: cached tokens of each sequence; token t of
 *                sequence b sits at slot t % block_size of physical block
 *                block_table[b][t / block_size]
 *   o            [batch, n_q_heads, head_dim] bf16, written
 *   lse          [batch, n_q_heads] fp32, written; may be NULL
 *   workspace    device scratch of at least attn_decode_workspace_bytes(...)
 *                bytes, 16-byte aligned (ATTN_ERR_ALIGN otherwise; torch
 *                allocations are 256-byte aligned); its contents on entry do not
 *                matter.  Calls that overlap in time (on different streams)
 *                need workspaces of their own.
 *
 * Every cached key of a sequence is visible to its query.  Sequence b's keys
 * are cut into `splits` chunks of equal length (a multiple of block_size,
 * the last one shorter or empty); each chunk is one partial, merged with the
 * log-sum-exp formula.  The result does not depend on the number of splits
 * beyond fp32 rounding.  Cache slots past ctx_lens[b] are never read, so
 * they may hold anything, NaN included.
 *
 * Supported: head_dim 64 or 128; block_size 16; n_q_heads / n_kv_heads <= 256;
 * num_splits in [1, ATTN_MAX_SPLITS] or <= 0 for the library's choice;
 * batch * n_kv_heads * splits < 2^31 (ATTN_ERR_SHAPE otherwise; with several
 * new tokens, times the groups of up to 64 (head, token) columns).
 * ctx_lens[b] == 0 gives O = 0, lse = -inf.
 * Device-side contract violations do not fault: a sequence whose ctx_lens
 * entry is negative or exceeds max_blocks_per_seq * block_size, or whose
 * needed block ids fall outside [0, num_blocks), gets NaN in o and lse.
 * Returns ATTN_ERR_WORKSPACE if workspace is NULL or workspace_bytes is too
 * small, and the other codes as for attn_prefill.
 */
attn_status_t attn_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *block_table, const int32_t *ctx_lens,
                                void *o, float *lse,
                                int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                int num_blocks, int block_size, int max_blocks_per_seq,
                                int num_splits, float scale,
                                void *workspace, size_t workspace_bytes,
                                attn_stream_t stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged without a caller-provided
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * arguments and results are those of attn_decode_paged with the workspace
 * arguments removed; the same kernels run with the same split count, so the
 * outputs are bit-identical to attn_decode_paged's.
 *
 * The workspace is a library-held array of ATTN_STATIC_SCRATCH_BYTES in
 * device memory, one per GPU the library runs on, held until the process
 * ends.  The call allocates nothing (no hipMalloc, no library allocator); the
 * first call on a device looks the array's device address up once.  Nothing
 * in the array has to start at zero: every partial is written before it is
 * read, and the work counter is reset by the kernel itself.  Every call on a
 * GPU shares that GPU's array and finds it as the last call left it, so calls
 * that overlap in time on one GPU (different streams, or several host
 * threads) RACE and give undefined results; serialise them, or use
 * attn_decode_paged with a workspace each.
 *
 * Returns ATTN_ERR_WORKSPACE, without touching the device, when
 * attn_decode_workspace_bytes(...) for these arguments exceeds
 * ATTN_STATIC_SCRATCH_BYTES (32 MiB: batch 64 with 32 query heads at
 * head_dim 128 fits up to 31 splits; batch 4 with 64 query heads and 64
 * splits takes 8.4 MB); ATTN_ERR_LAUNCH if the array's
 * address cannot be obtained; otherwise the codes of attn_decode_paged.
 */
#define ATTN_STATIC_SCRATCH_BYTES (32u << 20)

attn_status_t attn_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *block_table, const int32_t *ctx_lens,
                                        void *o, float *lse,
                                        int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                        int num_blocks, int block_size, int max_blocks_per_seq,
                                        int num_splits, float scale, attn_stream_t stream);

/*
 * attn_decode_paged_multi -- seqlen_q new query tokens per sequence over a
 * paged KV cache that already holds their keys: the verification step of
 * speculative decoding, where the draft tokens are checked in one pass
 * ("推理加速" interview notes, section speculative decoding: the target
 * model checks several draft tokens at once; "GPU Kernel 调度：大模型推理的
 * 拐点 2026", paragraph on the coupling of speculative decoding with
 * Flash-Decoding).  Same split-KV scheme and partial merge as
 * attn_decode_paged; the seqlen_q tokens share every K/V read.
 *
 *   q            [batch, seqlen_q, n_q_heads, head_dim]             bf16
 *   o            [batch, seqlen_q, n_q_heads, head_dim]             bf16, written
 *   lse          [batch, n_q_heads, seqlen_q] fp32, written; may be NULL
 *   workspace    attn_decode_multi_workspace_bytes(...) bytes, 16-byte aligned
 *   other arguments as for attn_decode_paged.
 *
 * Token t (0-based) of sequence b sits at position ctx_lens[b] - seqlen_q + t
 * and sees the keys at positions <= ctx_lens[b] - seqlen_q + t (causal among
 * the new tokens; the result equals attn_prefill_paged with the same
 * arguments).  A token with no visible key gets O = 0, lse = -inf.
 * Supported: (n_q_heads / n_kv_heads) * seqlen_q <= 256, plus the limits of
 * attn_decode_paged; seqlen_q == 1 is attn_decode_paged.
 *
 * num_splits <= 0 with seqlen_q > 1: the library's choice, again from the
 * arguments alone.  Each chunk writes a partial output per (token, query
 * head); with C = (n_q_heads / n_kv_heads) * seqlen_q:
 *   C <= 32: chunks of about 2048 * min(4, max(1, C / 4)) tokens of the
 *     longest sequence the table can hold, and more chunks (none shorter
 *     than 256 tokens) until about 256 items (chunk, sequence, KV head,
 *     group of up to 64 columns) occupy the GPU; for tables of more than
 *     4096 tokens and at least half as many workgroups as compute units,
 *     about four items per compute unit instead;
 *   C > 32: about two items per compute unit (four from half as many
 *     workgroups as compute units on), with chunks of at least 256 tokens
 *     and at least batch * n_q_heads * seqlen_q / 16 tokens.
 * attn_decode_multi_workspace_bytes sizes the workspace for the same choice.
 */
attn_status_t attn_decode_paged_multi(const void *q, const void *k_cache, const void *v_cache,
                                      const int32_t *block_table, const int32_t *ctx_lens,
                                      void *o, float *lse,
                                      int batch, int seqlen_q, int n_q_heads, int n_kv_heads,
                                      int head_dim, int num_blocks, int block_size,
                                      int max_blocks_per_seq, int num_splits, float scale,
                                      void *workspace, size_t workspace_bytes,
                                      attn_stream_t stream);

/*
 * attn_decode_paged_fp8 -- attn_decode_paged_multi over an 8-bit KV cache:
 * half the bytes per cached token, for decode steps limited by the bandwidth
 * of reading the cache ("5.2 推理加速的未来趋势", co-design layer: low-precision
 * KV caches as a lever on memory traffic; "推理加速" interview notes,
 * techniques table: KV-cache quantisation).  The pages fix no format; this
 * library reads OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, subnormals, 0x7F / 0xFF = NaN, no infinities, largest
 * finite value 448) with one scale per tensor:
 *     K = e4m3(k_cache) * k_scale,   V = e4m3(v_cache) * v_scale.
 *
 *   k_cache, v_cache  [num_blocks, block_size, n_kv_heads, head_dim] uint8
 *                     e4m3 codes
 *   k_scale, v_scale  finite dequantisation scales (ATTN_ERR_SHAPE otherwise)
 *   everything else as for attn_decode_paged_multi, including the workspace
 *   (attn_decode_multi_workspace_bytes).
 *
 * The codes are widened exactly to bf16 for the matrix-core products;
 * k_scale is folded into the score scale and v_scale applied to the fp32
 * partial outputs.
 */
attn_status_t attn_decode_paged_fp8(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_table, const int32_t *ctx_lens,
                                    void *o, float *lse,
                                    int batch, int seqlen_q, int n_q_heads, int n_kv_heads,
                                    int head_dim, int num_blocks, int block_size,
                                    int max_blocks_per_seq, int num_splits, float scale,
                                    float k_scale, float v_scale,
                                    void *workspace, size_t workspace_bytes,
                                    attn_stream_t stream);

/*
 * attn_decode_multi_workspace_bytes -- workspace of attn_decode_paged_multi:
 * partial outputs [batch, seqlen_q, n_q_heads, splits, head_dim] fp32, then
 * their log-sum-exps [batch, seqlen_q, n_q_heads, splits] fp32, with splits
 * the count attn_decode_paged_multi uses for these arguments
 * (attn_decode_num_splits when seqlen_q == 1), then 256 bytes of scheduling
 * state as for attn_decode_workspace_bytes.  Returns 0 for invalid
 * arguments.
 */
size_t attn_decode_multi_workspace_bytes(int batch, int seqlen_q, int n_q_heads, int n_kv_heads,
                                         int head_dim, int max_blocks_per_seq, int block_size,
                                         int num_splits);

/* Human-readable name of a status code (static storage, never NULL).  Part
 * of the boundary's plumbing: the pages define no error model, so the codes
 * and their names are this library's own. */
const char *attn_status_string(attn_status_t status);

/* ABI version of this header: (major << 16) | minor. */
int attn_abi_version(void);

#define ATTN_ABI_VERSION ((1 << 16) | 5)

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
