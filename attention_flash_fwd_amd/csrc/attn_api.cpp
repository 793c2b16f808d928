// attn_api.cpp -- the C ABI of libattn.so (declared in include/attn.h).
//
// Every argument is checked on the host before any HIP call; a rejected call
// enqueues nothing and touches no output.  Accepted calls enqueue their
// kernels on the caller's stream and return without synchronising.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "kernels.hpp"

namespace {

constexpr long long kMaxElems = 1LL << 31;   // per-tensor element limit of the prefill path
constexpr int kBlockSize = 16;
constexpr int kMaxColumns = 256;     // (query heads per KV head) x (new tokens) in paged decode
constexpr float kLog2e = 1.44269504088896340736f;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

attn_status_t check_prefill(const void *q, const void *k, const void *v, const void *o,
                            const float *lse, int B, int Sq, int Sk, int Hq, int Hkv, int D,
                            attn_dtype_t dtype)
{
    if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return ATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if ((long long)B * Sq * Hq * D >= kMaxElems || (long long)B * Sk * Hkv * D >= kMaxElems)
        return ATTN_ERR_SHAPE;
    if (B == 0 || Sq == 0) return ATTN_OK;
    if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
    if (Sk > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, 16) || !aligned(v, 16)) return ATTN_ERR_ALIGN;
    if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

// Chunks per sequence for decode: explicit, or the library's choice from the
// host-side arguments alone (never device data).  Chunks of about 2048
// tokens of the longest possible sequence keep each workgroup's stream long
// and the partial-output traffic small; for short contexts or few
// (sequence, KV head) pairs, more chunks (down to 256 tokens) are used until
// about 256 items, one per compute unit, cover the GPU.  (Measured on
// MI355X: batch 64 with contexts up to 32K is best at 12-16 chunks, batch 4
// at 128K at 64; 32 sequences of 1024 tokens at one chunk, 24.5 us against
// 37 us at the four that a 2048-item target gave.)
constexpr long long kFillItems = 256;
// Below this many tokens (the longest sequence the table can hold), one
// chunk per sequence: the Flash-Decoding threshold of "GPU Kernel 调度：大模型
// 推理的拐点 2026" (advice 2 and checklist item 2: below about 1024 tokens
// splitting is slower than not splitting).  The split-count sweep on MI355X
// (bench.py --split-sweep) agrees: at 512 tokens every split count is within
// a microsecond of one chunk or slower (batch 16: 14.1 us with one chunk,
// 15.9 us with two), while from 1024 tokens on, batches of 1-4 sequences
// decode 33-39% faster split.
constexpr long long kSplitThresholdTokens = 1024;
// Up to this many tokens, when one chunk per sequence already gives at least
// a quarter of the items that would fill the GPU twice, two chunks are not
// worth their merge.  Measured on MI355X, 16 sequences (32 query / 8 KV
// heads, D 128): one new token, 1024 tokens 16.8 us with one chunk against
// 20.4 us with two, 2048 tokens 26.4 against 28.5, 4096 tokens 44.7 against
// 47.2; 2 to 8 new tokens at 1024 tokens 17.0-21.5 against 20.8-26.0 us, at
// 4096 tokens within -11% to +3%.  With 64 sequences two chunks stay (4096
// tokens: 185 against 190 us).
constexpr long long kShortTokens = 4096;
// The same rule for one new token stops at 2048 tokens: with lengths drawn
// from 512 to 4096 tokens, 16 sequences took 38.1 us with one chunk against
// 30.5 us with two (equal lengths of 4096: 44.7 against 48.0 us).
constexpr long long kShortTokensOne = 2048;

int resolve_splits(int batch, int n_kv_heads, int max_blocks, int block_size, int num_splits)
{
    if (num_splits >= 1) return num_splits <= ATTN_MAX_SPLITS ? num_splits : 0;
    const long long max_tokens = (long long)max_blocks * block_size;
    const long long units = (long long)batch * n_kv_heads;
    if (units <= 0 || max_tokens < kSplitThresholdTokens) return 1;
    const long long by_length = (max_tokens + 2047) / 2048;
    // About one (chunk, sequence, KV head) item per compute unit: below
    // that, more chunks pay off; above it, each extra chunk costs more (its
    // partials and, from two chunks on, the merge kernel) than it gains.
    const long long by_fill = std::min((kFillItems + units - 1) / units, (max_tokens + 255) / 256);
    long long s = std::max(by_length, by_fill);
    // Two chunks of a short context do not pay for the merge they bring:
    // one chunk writes its result directly (see kShortTokens).
    if (s == 2 && max_tokens <= kShortTokensOne && units < 2 * kFillItems) s = 1;
    // The decode kernel switches to items of four KV heads (one per wave)
    // when they give at least one item per compute unit with chunks of at
    // most 2048 tokens.  When the call already splits and at most doubling
    // the count gives two such items per compute unit (chunks still of 256
    // tokens or more), take it: with two, the longest-first order balances
    // batches of mixed lengths, which one item per compute unit cannot
    // (lengths drawn from 512 up to 4096 tokens, 64 sequences: 4 chunks
    // 110.7 us, 2 chunks 127.1 us; up to 8192 tokens, 16 sequences: 8 chunks
    // (one item per compute unit) 50.1 us against 45.2 us with 4).  Equal
    // lengths lose a little against one item per compute unit (16 x 8192
    // tokens: 102.9 us at 4 chunks against 97.3 at 8).  One-chunk calls stay
    // so (batch 64 at 1024 and 2048 tokens: 2 chunks were 1-7% slower).
    if (s >= 2 && n_kv_heads % 4 == 0) {
        const long long groups = (long long)batch * (n_kv_heads / 4);
        const long long cus = attn::compute_units();
        const long long s4 = std::max(s, (2 * cus + groups - 1) / groups);
        if (s4 <= 2 * s && s4 <= (max_tokens + 255) / 256) s = s4;
    }
    if (s > ATTN_MAX_SPLITS) s = ATTN_MAX_SPLITS;
    if (s < 1) s = 1;
    return (int)s;
}

// Chunks per sequence with seqlen_q new tokens per sequence.  One token:
// resolve_splits.  Several, with up to 32 columns C = (n_q_heads /
// n_kv_heads) * seqlen_q: every chunk writes a partial output per (token,
// query head), so the partial traffic grows with C, and the chunks are
// longer, about 2048 * min(4, max(1, C / 4)) tokens of the longest
// sequence.  More chunks (none shorter than 256 tokens) are added until
// about 256 items, one per compute unit and counted with the column-tile
// groups, occupy the GPU (as for one token; short contexts at 2-8 tokens
// measured best there, e.g. 32 sequences of 1024 tokens at one chunk, 25 us
// against 35 us at the two a 512 target gave), or, for longer tables and
// larger calls, about four items per compute unit (below).  Against the
// single-token rule (MI355X): batch 64 with contexts up to 32K, 2-8 tokens,
// 3-5% faster; batch 4 at 128K, 8 tokens, 14% faster, 2-4 tokens within 1%.
int resolve_splits_multi(int batch, int seqlen_q, int n_q_heads, int n_kv_heads, int max_blocks,
                         int block_size, int num_splits)
{
    if (num_splits >= 1 || seqlen_q <= 1 || n_kv_heads <= 0)
        return resolve_splits(batch, n_kv_heads, max_blocks, block_size, num_splits);
    const long long max_tokens = (long long)max_blocks * block_size;
    const long long units = (long long)batch * n_kv_heads;
    if (units <= 0 || max_tokens <= 0) return 1;
    const long long cols = (long long)(n_q_heads / n_kv_heads) * seqlen_q;
    if (cols > 32) {
        // From 33 columns on the workgroups are wide (64 or 128 columns) and
        // each token costs them several times the matrix work of the narrow
        // tiles, so the count follows the workgroups rather than the tokens.
        // The kernel keeps two workgroups per compute unit resident and hands
        // out items longest sequence first; the count aims at two items per
        // compute unit for calls of fewer workgroups than half the compute
        // units, and at four otherwise (two rounds, which the longest-first
        // order balances when the lengths differ), with chunks no shorter
        // than 256 tokens or one token per sixteen partial rows (batch x
        // query heads x new tokens) the call writes.  Measured on MI355X at
        // 32 query / 8 KV heads, D 128, 16 and 32 new tokens, 4-64 sequences
        // of up to 8192 or 32768 tokens: with lengths drawn from 512 up, on
        // average within 1% of the best explicit count and at most 7% off
        // (the count that best fits equal lengths was up to 51% off there);
        // with equal lengths on average within 5% and at most 14% off (64 x
        // 8192 tokens at 32 new tokens, where one chunk is best).
        const long long per_wg = cols <= 64 ? 64 : 128;
        const long long wgs = units * ((cols + per_wg - 1) / per_wg);
        const long long cus = attn::compute_units();
        const long long items = (2 * wgs < cus ? 2 : 4) * cus;
        const long long min_chunk = std::max<long long>(256, units * cols / 16);
        long long s = std::min(std::max(1LL, items / wgs), std::max(1LL, max_tokens / min_chunk));
        if (s > ATTN_MAX_SPLITS) s = ATTN_MAX_SPLITS;
        return (int)s;
    }
    const long long f = std::min<long long>(4, std::max<long long>(1, cols / 4));
    const long long groups = ((cols + 15) / 16 + 3) / 4;     // workgroups per (chunk, sequence, KV head)
    const long long by_length = (max_tokens + 2048 * f - 1) / (2048 * f);
    const long long wgs = units * groups;
    // Past kShortTokens, calls of at least half as many workgroups as
    // compute units aim at four items per compute unit, as the wide path
    // does: with the longest-first item order that balances batches of mixed
    // lengths.  Measured on MI355X (32 query / 8 KV heads, D 128, 2-8 new
    // tokens, 16-64 sequences, lengths drawn from 512 up to 16384 or 32768
    // tokens): one chunk at 32 sequences of up to 16384 tokens took 230 us
    // with 4 new tokens against 165 us with four chunks; with equal lengths
    // the count costs up to 18% against the best (32 x 8192 tokens, 8 new
    // tokens: 231 against 196 us with one chunk).
    const long long cus = attn::compute_units();
    long long by_fill;
    if (max_tokens > kShortTokens && 2 * wgs >= cus)
        by_fill = std::max(1LL, 4 * cus / wgs);
    else
        by_fill = std::min((kFillItems + wgs - 1) / wgs, (max_tokens + 255) / 256);
    long long s = std::max(by_length, by_fill);
    // Two chunks of a short context do not pay for their merge (as for one
    // token).
    if (s == 2 && max_tokens <= kShortTokens && wgs < 2 * kFillItems) s = 1;
    if (s > ATTN_MAX_SPLITS) s = ATTN_MAX_SPLITS;
    if (s < 1) s = 1;
    return (int)s;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t part_o_bytes(int B, int Hq, int D, int S) { return align_up((size_t)B * Hq * S * D * sizeof(float), 256); }
size_t part_lse_bytes(int B, int Hq, int S) { return align_up((size_t)B * Hq * S * sizeof(float), 256); }
constexpr size_t kSchedBytes = 256;     // the split kernel's work counter, after the partials

}  // namespace

namespace attn {

int compute_units()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

}  // namespace attn

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char *attn_status_string(attn_status_t s)
{
    switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_SHAPE: return "invalid shape";
    case ATTN_ERR_DTYPE: return "invalid dtype";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

attn_status_t attn_prefill(const void *q, const void *k, const void *v, void *o, float *lse,
                           int batch, int seqlen_q, int seqlen_k, int n_q_heads, int n_kv_heads,
                           int head_dim, int causal, float scale, attn_dtype_t dtype,
                           attn_stream_t stream)
{
    attn_status_t st = check_prefill(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_q_heads,
                                     n_kv_heads, head_dim, dtype);
    if (st != ATTN_OK || batch == 0 || seqlen_q == 0) return st;

    attn::PrefillArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = batch;
    a.Sq = seqlen_q;
    a.Sk = seqlen_k;
    a.Hq = n_q_heads;
    a.Hkv = n_kv_heads;
    a.scale_log2 = scale * kLog2e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = dtype == ATTN_BF16 ? attn::launch_prefill_bf16(a, head_dim, causal != 0, s)
                                      : attn::launch_prefill_f32(a, head_dim, causal != 0, s);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_prefill_paged(const void *q, const void *k_cache, const void *v_cache,
                                 const int32_t *block_table, const int32_t *ctx_lens,
                                 void *o, float *lse,
                                 int batch, int seqlen_q, int n_q_heads, int n_kv_heads, int head_dim,
                                 int num_blocks, int block_size, int max_blocks_per_seq,
                                 int causal, float scale, attn_stream_t stream)
{
    if (batch < 0 || seqlen_q < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
        num_blocks < 0 || max_blocks_per_seq < 0 || block_size <= 0)
        return ATTN_ERR_SHAPE;
    if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
    if (block_size != kBlockSize) return ATTN_ERR_UNSUPPORTED;
    if ((long long)batch * seqlen_q * n_q_heads * head_dim >= kMaxElems) return ATTN_ERR_SHAPE;
    if ((long long)max_blocks_per_seq * block_size >= kMaxElems) return ATTN_ERR_SHAPE;
    // One cache block of one KV head must stay addressable by 32-bit offsets.
    if ((long long)block_size * n_kv_heads * head_dim * 2 >= (1LL << 31)) return ATTN_ERR_SHAPE;
    if (batch == 0 || seqlen_q == 0) return ATTN_OK;
    if (q == nullptr || o == nullptr || block_table == nullptr || ctx_lens == nullptr)
        return ATTN_ERR_NULL;
    if (num_blocks > 0 && (k_cache == nullptr || v_cache == nullptr)) return ATTN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
        return ATTN_ERR_ALIGN;
    if (!aligned(block_table, 4) || !aligned(ctx_lens, 4)) return ATTN_ERR_ALIGN;
    if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_ALIGN;

    attn::PrefillArgs a = {};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.o = o;
    a.lse = lse;
    a.B = batch;
    a.Sq = seqlen_q;
    a.Sk = 0;
    a.Hq = n_q_heads;
    a.Hkv = n_kv_heads;
    a.scale_log2 = scale * kLog2e;
    a.block_table = block_table;
    a.ctx_lens = ctx_lens;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks_per_seq;
    hipError_t e = attn::launch_prefill_paged_bf16(a, head_dim, causal != 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_decode_num_splits(int batch, int n_kv_heads, int max_blocks_per_seq, int block_size,
                           int num_splits)
{
    if (batch < 0 || n_kv_heads <= 0 || max_blocks_per_seq < 0 || block_size <= 0) return 0;
    return resolve_splits(batch, n_kv_heads, max_blocks_per_seq, block_size, num_splits);
}

size_t attn_decode_multi_workspace_bytes(int batch, int seqlen_q, int n_q_heads, int n_kv_heads,
                                         int head_dim, int max_blocks_per_seq, int block_size,
                                         int num_splits)
{
    if (batch < 0 || seqlen_q <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0) return 0;
    if (max_blocks_per_seq < 0 || block_size <= 0) return 0;
    const int S = resolve_splits_multi(batch, seqlen_q, n_q_heads, n_kv_heads, max_blocks_per_seq, block_size,
                                       num_splits);
    if (S <= 0) return 0;
    const int rows = batch * seqlen_q;
    return part_o_bytes(rows, n_q_heads, head_dim, S) + part_lse_bytes(rows, n_q_heads, S) + kSchedBytes;
}

size_t attn_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                   int max_blocks_per_seq, int block_size, int num_splits)
{
    return attn_decode_multi_workspace_bytes(batch, 1, n_q_heads, n_kv_heads, head_dim,
                                             max_blocks_per_seq, block_size, num_splits);
}

}  // extern "C"

namespace {

// Validation and launch shared by the three paged-decode entry points.
attn_status_t decode_common(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_table, const int32_t *ctx_lens, void *o, float *lse,
                            int batch, int seqlen_q, int n_q_heads, int n_kv_heads, int head_dim,
                            int num_blocks, int block_size, int max_blocks_per_seq, int num_splits,
                            float scale, bool kv_fp8, float k_scale, float v_scale,
                            void *workspace, size_t workspace_bytes, attn_stream_t stream)
{
    if (batch < 0 || seqlen_q <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
        num_blocks < 0 || max_blocks_per_seq < 0 || block_size <= 0)
        return ATTN_ERR_SHAPE;
    if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
    if (block_size != kBlockSize) return ATTN_ERR_UNSUPPORTED;
    if ((long long)(n_q_heads / n_kv_heads) * seqlen_q > kMaxColumns) return ATTN_ERR_UNSUPPORTED;
    if (num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_UNSUPPORTED;
    if (kv_fp8 && !(std::isfinite(k_scale) && std::isfinite(v_scale))) return ATTN_ERR_SHAPE;
    if ((long long)max_blocks_per_seq * block_size >= kMaxElems) return ATTN_ERR_SHAPE;
    if ((long long)batch * seqlen_q * n_q_heads * head_dim >= kMaxElems) return ATTN_ERR_SHAPE;
    if ((long long)block_size * n_kv_heads * head_dim * 2 >= (1LL << 31)) return ATTN_ERR_SHAPE;
    if (batch == 0) return ATTN_OK;
    if (q == nullptr || o == nullptr || block_table == nullptr || ctx_lens == nullptr)
        return ATTN_ERR_NULL;
    if (num_blocks > 0 && (k_cache == nullptr || v_cache == nullptr)) return ATTN_ERR_NULL;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
        return ATTN_ERR_ALIGN;
    if (!aligned(block_table, 4) || !aligned(ctx_lens, 4)) return ATTN_ERR_ALIGN;
    if (lse != nullptr && !aligned(lse, 4)) return ATTN_ERR_ALIGN;

    const int S = resolve_splits_multi(batch, seqlen_q, n_q_heads, n_kv_heads, max_blocks_per_seq, block_size,
                                       num_splits);
    // Split-kernel work items (chunk, KV head, sequence, group of up to 4
    // column tiles of 16) are numbered in 32 bits.
    const long long col_tiles = ((long long)(n_q_heads / n_kv_heads) * seqlen_q + 15) / 16;
    if ((long long)batch * n_kv_heads * S * ((col_tiles + 3) / 4) >= (1LL << 31)) return ATTN_ERR_SHAPE;
    const size_t need = attn_decode_multi_workspace_bytes(batch, seqlen_q, n_q_heads, n_kv_heads, head_dim,
                                                          max_blocks_per_seq, block_size, num_splits);
    if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;

    attn::DecodeArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.ctx_lens = ctx_lens;
    a.part_o = static_cast<float *>(workspace);
    a.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                           part_o_bytes(batch * seqlen_q, n_q_heads, head_dim, S));
    a.work_ctr = reinterpret_cast<unsigned *>(static_cast<char *>(workspace) +
                                              part_o_bytes(batch * seqlen_q, n_q_heads, head_dim, S) +
                                              part_lse_bytes(batch * seqlen_q, n_q_heads, S));
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.B = batch;
    a.T = seqlen_q;
    a.Hq = n_q_heads;
    a.Hkv = n_kv_heads;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.splits = S;
    a.scale_log2 = scale * (kv_fp8 ? k_scale : 1.0f) * kLog2e;
    a.v_scale = kv_fp8 ? v_scale : 1.0f;
    hipError_t e = attn::launch_decode(a, head_dim, kv_fp8, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

attn_status_t attn_decode_paged_multi(const void *q, const void *k_cache, const void *v_cache,
                                      const int32_t *block_table, const int32_t *ctx_lens,
                                      void *o, float *lse,
                                      int batch, int seqlen_q, int n_q_heads, int n_kv_heads,
                                      int head_dim, int num_blocks, int block_size,
                                      int max_blocks_per_seq, int num_splits, float scale,
                                      void *workspace, size_t workspace_bytes,
                                      attn_stream_t stream)
{
    return decode_common(q, k_cache, v_cache, block_table, ctx_lens, o, lse, batch, seqlen_q, n_q_heads,
                         n_kv_heads, head_dim, num_blocks, block_size, max_blocks_per_seq, num_splits,
                         scale, false, 1.0f, 1.0f, workspace, workspace_bytes, stream);
}

attn_status_t attn_decode_paged_fp8(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_table, const int32_t *ctx_lens,
                                    void *o, float *lse,
                                    int batch, int seqlen_q, int n_q_heads, int n_kv_heads,
                                    int head_dim, int num_blocks, int block_size,
                                    int max_blocks_per_seq, int num_splits, float scale,
                                    float k_scale, float v_scale,
                                    void *workspace, size_t workspace_bytes,
                                    attn_stream_t stream)
{
    return decode_common(q, k_cache, v_cache, block_table, ctx_lens, o, lse, batch, seqlen_q, n_q_heads,
                         n_kv_heads, head_dim, num_blocks, block_size, max_blocks_per_seq, num_splits,
                         scale, true, k_scale, v_scale, workspace, workspace_bytes, stream);
}

attn_status_t attn_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *block_table, const int32_t *ctx_lens,
                                void *o, float *lse,
                                int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                int num_blocks, int block_size, int max_blocks_per_seq,
                                int num_splits, float scale,
                                void *workspace, size_t workspace_bytes,
                                attn_stream_t stream)
{
    return attn_decode_paged_multi(q, k_cache, v_cache, block_table, ctx_lens, o, lse, batch, 1,
                                   n_q_heads, n_kv_heads, head_dim, num_blocks, block_size,
                                   max_blocks_per_seq, num_splits, scale, workspace, workspace_bytes,
                                   stream);
}

attn_status_t attn_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *block_table, const int32_t *ctx_lens,
                                        void *o, float *lse,
                                        int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                        int num_blocks, int block_size, int max_blocks_per_seq,
                                        int num_splits, float scale, attn_stream_t stream)
{
    // The size check runs before anything touches the device.  A shape the
    // workspace rules reject (0 bytes) goes on to decode_common, which
    // returns the matching status code without launching.
    const size_t need = attn_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim,
                                                    max_blocks_per_seq, block_size, num_splits);
    if (need > ATTN_STATIC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0 && batch > 0) {
        ws = attn::static_scratch();
        if (ws == nullptr) return ATTN_ERR_LAUNCH;
    }
    return decode_common(q, k_cache, v_cache, block_table, ctx_lens, o, lse, batch, 1, n_q_heads,
                         n_kv_heads, head_dim, num_blocks, block_size, max_blocks_per_seq, num_splits,
                         scale, false, 1.0f, 1.0f, ws, ws != nullptr ? ATTN_STATIC_SCRATCH_BYTES : 0,
                         stream);
}

}  // extern "C"
