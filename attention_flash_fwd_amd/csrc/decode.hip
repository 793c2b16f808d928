// decode.hip -- attention of one (or a few) new tokens per sequence over a
// paged KV cache, Flash-Decoding style ("GPU Kernel 调度：大模型推理的拐点
// 2026", paragraphs on Flash Decoding and its cost: the cached K/V of a
// sequence is cut into chunks processed in parallel, each chunk yields a
// partial output with its log-sum-exp, and a small reduce kernel merges the
// partials with the online-softmax formula in fp32; chenyy20.com
// "抱infra脚", section Paged Attention: fixed-size blocks reached through a
// block table).
//
// Kernel 1, decode_split: a workgroup of four waves computes one (chunk, KV
//   head, sequence) item at a time (or, for one new token with enough work,
//   a (chunk, four KV heads, sequence) item: each wave then streams one
//   head's blocks of the whole chunk and writes its own result).  With one or two column tiles (below), as many workgroups as
//   the GPU holds stay resident and take items from a work counter in the
//   workspace; with more, each workgroup computes one item.  The G = Hq / Hkv query heads that share the KV head, times
//   the T new tokens of the sequence (T = 1 for plain decode, several for
//   speculative verification), are the columns of the matrix-core products,
//   so each K/V byte is read from HBM once for all of them.  The chunk's
//   16-token cache blocks are dealt round-robin to the waves.  Each wave
//   streams its blocks with LDS-direct buffer loads into a private two-slot
//   ring (the next block lands while the current one is computed) and keeps
//   its own running max, running sum and partial output.  Per block:
//     S^T (16 tokens x 16 columns) = K Q^T   4 x 16x16x32 bf16 MFMA
//     P = 2^(S - m), lazy rescale of (l, O) when the max grows by > 2^8
//     O^T (D x 16 columns)       += V^T P^T  D/16 x 16x16x16 bf16 MFMA
//   New token t sees the keys up to position ctx - T + t; that limit is only
//   checked on the blocks that reach past ctx - T.  More than 16 columns are
//   split over column tiles of 16; one workgroup computes up to four tiles
//   from the same LDS copy of each block (every K and V^T fragment it reads
//   feeds one product per tile), and more tiles than that go to several
//   workgroups.
//   The score accumulator of a lane (4 tokens of one head) is exactly the
//   B operand the 16x16x16 product wants, and the V^T operand comes from one
//   transposing LDS read per 16 rows of d.  Cache slots past the chunk end
//   are never fetched (their buffer offsets fall outside the block and read
//   as zero).  The four wave partials are merged in LDS and the chunk's
//   normalised output and log-sum-exp are written as fp32.
// Kernel 2, decode_combine: one wave per (sequence, token, query head) merges
//   the chunk partials: M = max lse_s, w_s = e^(lse_s - M),
//   O = sum w_s O_s / sum w_s, lse = M + ln sum w_s; O rounded to bf16.
//   With a single chunk the merge is the identity (w = 1), so the split
//   kernel writes O and lse itself and this kernel is not launched.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "gfx950.hpp"
#include "kernels.hpp"
#include "../../include/attn.h"

namespace attn {
namespace {

constexpr int kBS = 16;         // tokens per cache block
constexpr int kWaves = 4;
// 16-column tiles one split workgroup computes at most.  A tile holds its
// accumulator (D / 8 registers), its row statistics and, in registers, its
// Q operand (D / 16).  With D = 128, four tiles fit 256 registers only once
// their Q operands move to LDS (16 KiB, which with the 64 KiB ring still
// lets two workgroups share a CU).
constexpr int kMaxTiles = 4;
// Split workgroups take their items from a work counter (staying resident)
// for one or two column tiles; with more, each runs one item of a grid laid
// out over the XCDs.  Measured on MI355X: the counter gains 1-4% where a
// chunk is read in one pass, and loses up to 7% where several workgroups
// share a chunk's reads through L2.
template <int NCT>
constexpr bool dynamic_items() { return NCT <= 2; }

template <int D, int NCT>
constexpr bool qs_in_lds() { return D == 128 && NCT == 4; }
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRanked = 256;     // sequences ranked by length for the item order
constexpr uint32_t kOutside = 0x80000000u;   // buffer offset past any block: reads zero

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;

__device__ __forceinline__ f32x4_t mfma_16x16x16_bf16(u32x2_t a, u32x2_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                     __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}

// One cache block of one KV head in LDS: 16 token rows of D elements of EB
// bytes (2: bf16, 1: fp8 e4m3).  16-byte chunk c of row r holds global chunk
// c ^ swz(r), which keeps the row-wise K reads (16 bytes per lane for bf16, 8
// for fp8) and the transposing V reads free of bank conflicts.
template <int D, int EB = 2>
struct Geom {
    static constexpr int row_bytes = EB * D;
    static constexpr int rows_per_load = 1024 / row_bytes;   // rows one wave-wide DMA fills
    static constexpr int loads = kBS / rows_per_load;        // DMAs per block of K (or V)
    static constexpr int slot_bytes = kBS * row_bytes;
    __device__ static __forceinline__ int swz(int r)
    {
        if constexpr (EB == 2)
            return D == 128 ? (((r << 1) | (r >> 3)) & 15) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
        else   // rows of 128 or 64 bytes: spread the rows that share banks over the chunks
            return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
    }
};

// Per-wave state of the split kernel for one 16-column tile.
template <int D>
struct WaveState {
    u32x4_t qf[D / 32];         // Q^T operand: head l16, d = 32 kk + 8 g .. +8
    f32x4_t o[D / 16];          // O^T: head l16, d = 16 db + 4 g + v
    float m, l;
};

// Queue the K and V of one block into a slot.  `valid` rows (tokens) are
// fetched, the rest read as zero; voff[i] is this lane's offset in the block
// for its row of DMA i.
template <class Gm>
__device__ __forceinline__ void issue_block(const void *kc, const void *vc, long long phys,
                                            uint32_t blk_bytes, int valid, const uint32_t (&voff)[Gm::loads],
                                            int lane, uint8_t *ks, uint8_t *vs)
{
    const char *kb = reinterpret_cast<const char *>(kc) + phys * blk_bytes;
    const char *vb = reinterpret_cast<const char *>(vc) + phys * blk_bytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, blk_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, blk_bytes);
    const int row0 = lane / (Gm::row_bytes / 16);
#pragma unroll
    for (int i = 0; i < Gm::loads; ++i) {
        const uint32_t off = (i * Gm::rows_per_load + row0 < valid) ? voff[i] : kOutside;
        buffer_load_lds16(rk, ks + 1024 * i, off);
        buffer_load_lds16(rv, vs + 1024 * i, off);
    }
}

// Convert this wave's fp8 V block (slot layout Geom<D,1>) to bf16 in the
// scratch block cv (layout Geom<D,2>): lane L handles row L / 4, a quarter
// of its elements.
template <int D>
__device__ __forceinline__ void convert_v(const uint8_t *vs, uint8_t *cv, int lane)
{
    using G8 = Geom<D, 1>;
    using G16 = Geom<D, 2>;
    constexpr int CH = D / 64;                   // fp8 chunks (16 values) per lane
    const int r = lane >> 2, q4 = lane & 3;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int gc = q4 * CH + i;              // fp8 chunk: values 16 gc .. 16 gc + 15
        const u32x4_t x = *reinterpret_cast<const u32x4_t *>(vs + r * G8::row_bytes + ((gc ^ G8::swz(r)) << 4));
        const u32x2_t a0 = fp8x4_to_bf16(x[0]), a1 = fp8x4_to_bf16(x[1]);
        const u32x2_t a2 = fp8x4_to_bf16(x[2]), a3 = fp8x4_to_bf16(x[3]);
        const u32x4_t lo = {a0[0], a0[1], a1[0], a1[1]}, hi = {a2[0], a2[1], a3[0], a3[1]};
        *reinterpret_cast<u32x4_t *>(cv + r * G16::row_bytes + (((2 * gc) ^ G16::swz(r)) << 4)) = lo;
        *reinterpret_cast<u32x4_t *>(cv + r * G16::row_bytes + (((2 * gc + 1) ^ G16::swz(r)) << 4)) = hi;
    }
}

// One block: scores, online softmax, PV, for NCT column tiles at once.  ks
// holds K with EB-byte elements; vs holds V as bf16 (for fp8 caches, the
// converted scratch copy).  Each K fragment and each V^T fragment read from
// LDS feeds the products of every tile.  With QL the Q^T operands come from
// LDS (qs: this lane's fragment of tile 0, kk 0; the fragments of (c, kk)
// follow at a stride of 1 KiB) instead of w[c].qf.
// Tokens 4 g + v of the block at or past `valid` are masked; with `causal`
// set, so is every token past lim[c] (absolute position) for this lane's
// column of tile c (the causal limit of its query among several new tokens).
template <int D, int EB, int NCT, bool QL>
__device__ __forceinline__ void compute_block(const uint8_t *ks, const uint8_t *vs, lds_u8 *qs,
                                              int valid, bool causal, int tok0, const int (&lim)[NCT],
                                              float scale_log2, int l16, int g, WaveState<D> (&w)[NCT])
{
    using Gm = Geom<D, 2>;
    using GK = Geom<D, EB>;
    f32x4_t s[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) s[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
        const uint8_t *row = ks + l16 * GK::row_bytes;
        const int sw = GK::swz(l16);
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            u32x4_t kf;
            if constexpr (EB == 2) {
                kf = *reinterpret_cast<const u32x4_t *>(row + (((4 * kk + g) ^ sw) << 4));
            } else {
                // d = 32 kk + 8 g .. +8: 8 bytes of fp8 chunk 2 kk + g / 2.
                const u32x2_t x = *reinterpret_cast<const u32x2_t *>(row + (((2 * kk + (g >> 1)) ^ sw) << 4) + ((g & 1) << 3));
                const u32x2_t lo = fp8x4_to_bf16(x[0]), hi = fp8x4_to_bf16(x[1]);
                kf = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
                u32x4_t qop;
                if constexpr (QL)
                    qop = *reinterpret_cast<lds_u32x4 *>(qs + 1024 * (c * (D / 32) + kk));
                else
                    qop = w[c].qf[kk];
                s[c] = mfma_16x16x32_bf16(kf, qop, s[c]);
            }
        }
    }
    // V^T operand: lane (g, i) receives V[4 g + e][16 db + i], e = 0..3, from
    // the rows 4 g + l16 / 4 read by its group.  Read now, so that the
    // softmax below hides the reads' latency.
    u32x2_t vt[D / 16];
    {
        const int vr = 4 * g + (l16 >> 2);
        const uint8_t *vrow = vs + vr * Gm::row_bytes + ((l16 & 1) << 3);
        const int vsw = Gm::swz(vr);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            const int chunk = 2 * db + ((l16 & 3) >> 1);
            vt[db] = lds_read_tr16(reinterpret_cast<const uint16_t *>(vrow + ((chunk ^ vsw) << 4)));
        }
    }
    // Lane (g, l16) holds tokens 4 g + v of head l16; the four lanes l16 +
    // 16 g' hold the column's 16 tokens.  Masking only where the block ends
    // early or reaches past a causal limit (a uniform branch).  One branch
    // covers the lazy rescale of every tile, so the accumulators are touched
    // on a single path.
#pragma unroll
    for (int c = 0; c < NCT; ++c) s[c] *= scale_log2;
    if (valid < kBS || causal) {
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool vis = 4 * g + v < valid && (!causal || tok0 + 4 * g + v <= lim[c]);
                s[c][v] = vis ? s[c][v] : kNegInf;
            }
    }
    float m_new[NCT];
    bool grow_any = false;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
        // max over the column's tokens: in-lane, then across the wave's
        // quarters (v_permlane16_swap, v_permlane32_swap)
        float mx = fmaxf(fmaxf(s[c][0], s[c][1]), fmaxf(s[c][2], s[c][3]));
        mx = pair_max_quarters(mx);
        mx = pair_max_halves(mx);
        m_new[c] = fmaxf(w[c].m, mx);
        grow_any |= m_new[c] > w[c].m + 8.0f;
    }
    if (wave_any(grow_any)) {
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            const bool grow = m_new[c] > w[c].m + 8.0f;
            const float alpha = grow ? exp2_fast(w[c].m - m_new[c]) : 1.0f;
            w[c].m = grow ? m_new[c] : w[c].m;
            w[c].l *= alpha;
#pragma unroll
            for (int db = 0; db < D / 16; ++db) w[c].o[db] *= alpha;
        }
    }
    u32x2_t pk[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
        const float mref = (w[c].m == kNegInf) ? 0.f : w[c].m;
        float p[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            p[v] = exp2_fast(s[c][v] - mref);
            w[c].l += p[v];
        }
        pk[c] = u32x2_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int c = 0; c < NCT; ++c) w[c].o[db] = mfma_16x16x16_bf16(vt[db], pk[c], w[c].o[db]);
}

template <int D, int EB, int NCT, int HPI>
__global__ void __launch_bounds__(kThreads, 2) decode_split_kernel(DecodeArgs a)
{
    static_assert(HPI == 1 || (HPI == kWaves && NCT == 1), "heads per item: 1, or one per wave with one tile");
    using Gm = Geom<D, EB>;
    // Two ring slots per wave, K and V each in an array of its own so that the
    // compiler's wait for a slot's loads does not also wait for the other's.
    __shared__ __attribute__((aligned(1024))) uint8_t k_s0[kWaves][Gm::slot_bytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_s0[kWaves][Gm::slot_bytes];
    __shared__ __attribute__((aligned(1024))) uint8_t k_s1[kWaves][Gm::slot_bytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_s1[kWaves][Gm::slot_bytes];
    // One more area after the ring: for fp8 caches, each wave's V block
    // converted to bf16 (one block per wave); with QL, the Q^T operands of the
    // NCT tiles, shared by the four waves (1 KiB per (tile, kk): 16 bytes a
    // lane).  With neither, a token 16 bytes.
    constexpr bool QL = qs_in_lds<D, NCT>();
    constexpr int kCv = EB == 1 ? kWaves * Geom<D, 2>::slot_bytes : 0;
    constexpr int kQs = QL ? NCT * (D / 32) * 1024 : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t aux[kCv + kQs > 0 ? kCv + kQs : 16];
    uint8_t *const v_cv = aux;                          // [kWaves][block]
    uint8_t *const q_s = aux + kCv;

    const int wave = (int)uniform_u32(threadIdx.x >> 6);

    const int G = a.Hq / a.Hkv;
    const int T = a.T;                  // new tokens per sequence
    const int GT = G * T;               // matrix-core columns in use: (token, head) pairs
    // Work item -> (tile group, chunk, KV head, sequence).  Columns come in
    // tiles of 16; an item is NCT consecutive tiles computed from one pass
    // over its chunk.
    //  - One or two tiles (DYN): the workgroups stay resident.  Workgroup w
    //    runs item w first; the items past the grid come from a counter in
    //    the workspace, so that workgroups on a faster XCD take more of them.
    //    Workgroup 0 zeroes the counter as it starts.  Whatever the counter
    //    held before, no item is lost: a ticket taken before the reset
    //    either lies past the end (that workgroup stops early) or is issued
    //    again after it (the item is computed twice, with identical
    //    results), and workgroup 0 keeps taking tickets until the counter
    //    passes the last item.
    //  - More tiles: one item per workgroup.  Past NCT tiles, the groups of
    //    one (chunk, KV head, sequence) get ids 8 apart, so they run at the
    //    same time on the same XCD (ids go round-robin over the 8 XCDs) and
    //    share its L2 copy of the K/V blocks; a chunk is far larger than the
    //    L2 share of one workgroup, so groups run one after another would
    //    each read it from HBM.
    constexpr bool DYN = dynamic_items<NCT>();
    const int n_ct = (GT + 15) / 16;
    const int n_grp = (n_ct + NCT - 1) / NCT;
    const unsigned n_units = (unsigned)(a.B * (a.Hkv / HPI) * a.splits);
    // DYN: thread 0 takes the next item's ticket while the current item's
    // partials merge (hiding the atomic's latency) and passes the item id to
    // the four waves through an LDS word of its own.  One barrier per item
    // suffices: a wave reaches it only once done with the previous item, and
    // thread 0 writes the word again only after the item's own barriers,
    // which every wave passes after reading it.
    __shared__ unsigned item_slot[1];
    unsigned ticket = 0;                // thread 0: the ticket for the next item
    // A long item started late would set the kernel's end (with HPI > 1
    // each wave streams a whole chunk).  Items are therefore handed out
    // longest sequence first (list scheduling): each workgroup ranks the
    // sequences by length (ties by index, a permutation) into an LDS table
    // as it starts.  More sequences than the table holds keep their order.
    // (One-head items, lengths drawn from 512 up to 16384 or 32768 tokens,
    // 2-8 new tokens, 16-64 sequences: up to 11% faster than in index order;
    // bit-identical output.)
    __shared__ int16_t seq_order[DYN ? kMaxRanked : 1];
    __shared__ int ctx_s[DYN ? kMaxRanked : 1];
    const bool ranked = DYN && a.B <= kMaxRanked;
    if (ranked) {
        // Lengths staged in LDS, then compared with broadcast reads.
        for (int i = threadIdx.x; i < a.B; i += kThreads) ctx_s[i] = a.ctx_lens[i];
        __syncthreads();
        for (int i = threadIdx.x; i < a.B; i += kThreads) {
            const int ci = ctx_s[i];
            int r = 0;
#pragma unroll 8
            for (int j = 0; j < a.B; ++j) {
                const int cj = ctx_s[j];
                r += (cj > ci) | ((cj == ci) & (j < i));
            }
            seq_order[r] = (int16_t)i;
        }
        __syncthreads();
    }
    if (DYN && blockIdx.x == 0 && threadIdx.x == 0) atomicExch(a.work_ctr, 0u);
    for (int round = 0;; ++round) {
    int grp, unit;
    if constexpr (DYN) {
        const unsigned n_items = n_units * (unsigned)n_grp;
        unsigned item = blockIdx.x;
        if (round > 0) {
            // tickets 0, 1, ... stand for items gridDim.x, gridDim.x + 1, ...
            if (threadIdx.x == 0)
                item_slot[0] = ticket < n_items - gridDim.x ? gridDim.x + ticket : n_items;
            __syncthreads();
            item = uniform_u32(item_slot[0]);
        }
        if (item >= n_items) break;
        grp = (int)(item % (unsigned)n_grp);
        unit = (int)(item / (unsigned)n_grp);
    } else {
        if (round > 0) break;
        const int L = blockIdx.x, r8 = L >> 3;
        grp = r8 % n_grp;
        unit = (r8 / n_grp) * 8 + (L & 7);
        if (unit >= (int)n_units) break;            // padding of the id space (uniform)
    }
    // DYN: lane index through opaque(), so that the per-lane addresses below
    // are formed for each item, not hoisted out of the item loop into
    // registers held across it.
    const int lane = DYN ? opaque((int)(threadIdx.x & 63)) : (int)(threadIdx.x & 63);
    const int l16 = lane & 15, g = lane >> 4;
    // HPI = kWaves: the item is KV heads HPI j .. HPI j + HPI - 1 of the
    // chunk, wave w computing head HPI j + w over every block of the chunk,
    // so that the workgroup reads HPI adjacent head rows of each token at
    // about the same time.  HPI = 1: one KV head, its blocks dealt to the
    // waves.
    const int split = unit % a.splits;
    const int hk = ((unit / a.splits) % (a.Hkv / HPI)) * HPI + (HPI > 1 ? wave : 0);
    const int bq = unit / (a.splits * (a.Hkv / HPI));
    const int b = ranked ? (int)uniform_u32((uint32_t)seq_order[bq]) : bq;
    const int col_base = 16 * NCT * grp;            // first column of tile 0; tile c starts 16 c later

    // Sequence length through the scalar cache: everything derived from it
    // (chunk bounds, trip counts) stays wave-uniform.
    const int ctx = ((const int32_t __attribute__((address_space(4))) *)a.ctx_lens)[b];
    bool bad = ctx < 0 || ctx > a.max_blocks * kBS;
    int t_begin = 0, t_end = 0;
    if (!bad && ctx > 0) {
        const int per = (ctx + a.splits - 1) / a.splits;
        const int chunk = (per + kBS - 1) / kBS * kBS;
        t_begin = min(split * chunk, ctx);
        t_end = min(t_begin + chunk, ctx);
    }
    const int blk0 = t_begin / kBS;
    const int nblk = (t_end - t_begin + kBS - 1) / kBS;
    // This wave's blocks: chunk blocks first, first + kStride, ...
    constexpr int kStride = HPI > 1 ? 1 : kWaves;
    const int first = HPI > 1 ? 0 : wave;
    const int nmine = HPI > 1 ? nblk : (nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0);

    // Column col = t G + g holds query head hk G + g of new token t.  Columns
    // past G T (a ragged last tile, or whole tiles of the last group) read
    // the last valid one and are zeroed (no branch around the load); they
    // are never written out.
    WaveState<D> w[NCT];
    int lim[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
        const int want = col_base + 16 * c + l16;
        const bool hv = want < GT;
        const int col = min(want, GT - 1);
        const uint16_t *qp = a.q + (((size_t)b * T + col / G) * a.Hq + hk * G + col % G) * D + 8 * g;
        if (!QL || c % kWaves == wave) {   // with QL, wave c % 4 stages tile c
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                const u32x4_t x = *reinterpret_cast<const u32x4_t *>(qp + 32 * kk);
                const u32x4_t v = hv ? x : u32x4_t{0, 0, 0, 0};
                if constexpr (QL)
                    *reinterpret_cast<u32x4_t *>(q_s + 1024 * (c * (D / 32) + kk) + 16 * lane) = v;
                else
                    w[c].qf[kk] = v;
            }
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db) w[c].o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        w[c].m = kNegInf;
        w[c].l = 0.f;
        // New token t sees keys up to position ctx - T + t.
        lim[c] = ctx - T + col / G;
    }

    // Physical block ids come through the scalar cache (the table is read-only
    // here), one block ahead of their use, so that the loop issues no vector
    // loads besides the K/V streams and every wait for a slot is exact.
    const int32_t __attribute__((address_space(4))) *tb =
        (const int32_t __attribute__((address_space(4))) *)(a.block_table + (size_t)b * a.max_blocks + blk0 + first);
    int phys_next = nmine > 0 ? tb[0] : 0;

    // This lane's offset inside a block for each of its DMAs: row
    // i * rows_per_load + lane / chunks_per_row, chunk lane % chunks_per_row
    // filled from global chunk (lane % chunks_per_row) ^ swz(row).
    const uint32_t blk_bytes = (uint32_t)(kBS * a.Hkv * Gm::row_bytes);
    uint32_t voff[Gm::loads];
    {
        constexpr int cpr = Gm::row_bytes / 16;
#pragma unroll
        for (int i = 0; i < Gm::loads; ++i) {
            const int r = i * Gm::rows_per_load + lane / cpr;
            const int c = (lane % cpr) ^ Gm::swz(r);
            voff[i] = (uint32_t)(r * a.Hkv * Gm::row_bytes + hk * Gm::row_bytes + 16 * c);
        }
    }

    // Issue block j of this wave into a slot (j past the end: nothing fetched).
    auto issue = [&](int j, uint8_t *ks, uint8_t *vs) __attribute__((always_inline)) {
        long long phys = 0;
        int valid = 0;
        if (j < nmine) {
            const int p = phys_next;
            phys_next = j + 1 < nmine ? tb[kStride * (j + 1)] : 0;
            const int tok0 = (blk0 + first + kStride * j) * kBS;
            if (p < 0 || p >= a.num_blocks) {
                bad = true;
            } else {
                phys = p;
                valid = min(kBS, t_end - tok0);
            }
        }
        issue_block<Gm>(a.k_cache, a.v_cache, phys, blk_bytes, valid, voff, lane, ks, vs);
    };
    auto valid_rows = [&](int j) __attribute__((always_inline)) {
        return min(kBS, t_end - (blk0 + first + kStride * j) * kBS);
    };
    // Only blocks reaching past ctx - T need the causal check.
    auto tok0_of = [&](int j) __attribute__((always_inline)) { return (blk0 + first + kStride * j) * kBS; };
    auto causal_blk = [&](int j) __attribute__((always_inline)) { return T > 1 && tok0_of(j) + kBS - 1 > ctx - T; };

    // Every path through the loop issues the same loads in the same order,
    // so the wait before each slot's reads is exact.
    auto run = [&](const uint8_t *ks, const uint8_t *vs, int j) __attribute__((always_inline)) {
        const uint8_t *vb = vs;
        if constexpr (EB == 1) {
            convert_v<D>(vs, v_cv + wave * Geom<D, 2>::slot_bytes, lane);
            __builtin_amdgcn_wave_barrier();
            vb = v_cv + wave * Geom<D, 2>::slot_bytes;
        }
        // An LDS address the compiler cannot see through, so that it reads
        // the Q operands in every block instead of keeping them live.
        lds_u8 *qb = (lds_u8 *)(q_s + 16 * lane);
        if constexpr (QL) asm volatile("" : "+v"(qb));
        compute_block<D, EB, NCT, QL>(ks, vb, qb, valid_rows(j), causal_blk(j), tok0_of(j), lim, a.scale_log2, l16, g, w);
    };
    if constexpr (QL) __syncthreads();              // the staged Q operands are visible
    issue(0, k_s0[wave], v_s0[wave]);
    issue(1, k_s1[wave], v_s1[wave]);
    for (int j = 0; j < nmine; j += 2) {
        run(k_s0[wave], v_s0[wave], j);
        issue(j + 2, k_s0[wave], v_s0[wave]);
        if (j + 1 < nmine) run(k_s1[wave], v_s1[wave], j + 1);
        issue(j + 3, k_s1[wave], v_s1[wave]);
    }

    // Row sums: lanes g = 0..3 of a head hold disjoint tokens.
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
        w[c].l += __shfl_xor(w[c].l, 16);
        w[c].l += __shfl_xor(w[c].l, 32);
    }

    // Merge the four wave partials in LDS, one column tile at a time.  The
    // ring is free once every wave has drained its loads (the trailing ones
    // past the chunk end fetch nothing but still write zeros) and passed the
    // barrier.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (DYN && threadIdx.x == 0) ticket = atomicAdd(a.work_ctr, 1u);
    if constexpr (HPI > 1) {
        // Each wave holds its head's whole chunk: normalise and write its
        // columns straight from the accumulators (lane (g, l16): column l16,
        // d = 16 db + 4 g .. +3).  Every wave reads the same block ids, so
        // they agree on `bad`.
        if (l16 < GT) {
            const float L = w[0].l;
            const float inv = bad ? __builtin_nanf("") : (L > 0.f ? a.v_scale / L : 0.f);
            const float lse = bad ? __builtin_nanf("") : (L > 0.f ? (w[0].m + __log2f(L)) * kLn2 : kNegInf);
            const int tq = l16 / G, hq = hk * G + l16 % G;
            const size_t orow = ((size_t)b * T + tq) * a.Hq + hq;
            if (a.splits == 1) {
                uint16_t *dst = a.o + orow * D + 4 * g;
#pragma unroll
                for (int db = 0; db < D / 16; ++db) {
                    const f32x4_t x = w[0].o[db] * inv;
                    *reinterpret_cast<u32x2_t *>(dst + 16 * db) = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                }
                if (g == 0 && a.lse != nullptr) a.lse[((size_t)b * a.Hq + hq) * T + tq] = lse;
            } else {
                const size_t row = orow * a.splits + split;
                float *dst = a.part_o + row * D + 4 * g;
#pragma unroll
                for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4_t *>(dst + 16 * db) = w[0].o[db] * inv;
                if (g == 0) a.part_lse[row] = lse;
            }
        }
        continue;
    }
    // Wave w's partial O (16 columns x D fp32): bf16 caches put two waves in
    // each of k_s0 / v_s0, fp8 caches one wave in each of the four slots.
    auto merge_area = [&](int v) __attribute__((always_inline)) -> float * {
        if constexpr (EB == 2)
            return reinterpret_cast<float *>(v < 2 ? &k_s0[0][0] : &v_s0[0][0]) + (v & 1) * 16 * D;
        else
            return reinterpret_cast<float *>(v == 0 ? &k_s0[0][0] : v == 1 ? &v_s0[0][0] : v == 2 ? &k_s1[0][0] : &v_s1[0][0]);
    };
    float *mo = merge_area(wave);
    float *ml = reinterpret_cast<float *>(EB == 2 ? &k_s1[0][0] : v_cv);   // [wave][16] m, then l
    int *flags = reinterpret_cast<int *>(ml + 2 * kWaves * 16);            // [wave] a bad block id seen
    {
        const bool wbad = wave_any(bad);
        if (lane == 0) flags[wave] = wbad ? 1 : 0;
    }
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
        const int col0 = col_base + 16 * c;
        if (col0 >= GT) break;                      // uniform: the rest of the group is past the columns
        const int NC = min(16, GT - col0);          // columns of this tile
        if (c > 0) __syncthreads();                 // the previous tile's readers are done
        if (g == 0) {
            ml[wave * 16 + l16] = w[c].m;
            ml[kWaves * 16 + wave * 16 + l16] = w[c].l;
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
            *reinterpret_cast<f32x4_t *>(mo + l16 * D + 16 * db + 4 * g) = w[c].o[db];
        __syncthreads();
        bool any_bad = false;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) any_bad |= flags[v] != 0;

        // Thread (column hh, d range dq): 16 threads per column, D / 16
        // consecutive d each; the column's wave weights are computed once.
        // Waves that saw no visible key have m = -inf, l = 0 and O = 0, and
        // add exact zeros.
        constexpr int DPT = D / 16;
        static_assert(kThreads == 16 * 16, "one thread per (column, d range)");
        const int hh = threadIdx.x >> 4, dq = threadIdx.x & 15;
        if (hh < NC) {
            float M = kNegInf;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) M = fmaxf(M, ml[v * 16 + hh]);
            float sc[kWaves];
            float Ls = 0.f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                const float mv = ml[v * 16 + hh];
                sc[v] = mv == kNegInf ? 0.f : exp2_fast(mv - M);
                Ls += ml[kWaves * 16 + v * 16 + hh] * sc[v];
            }
            float o[DPT];
#pragma unroll
            for (int i = 0; i < DPT; ++i) o[i] = 0.f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                const float *src = merge_area(v) + hh * D + dq * DPT;
#pragma unroll
                for (int i = 0; i < DPT; i += 4) {
                    const f32x4_t x = *reinterpret_cast<const f32x4_t *>(src + i);
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[i + e] += x[e] * sc[v];
                }
            }
            const int gcol = col0 + hh;
            const int tq = gcol / G, hq = hk * G + gcol % G;        // new token, query head
            const size_t orow = ((size_t)b * T + tq) * a.Hq + hq;
#pragma unroll
            for (int i = 0; i < DPT; ++i) {
                o[i] = Ls > 0.f ? o[i] / Ls * a.v_scale : 0.f;
                if (any_bad) o[i] = __builtin_nanf("");
            }
            const float lse = any_bad ? __builtin_nanf("") : (Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : kNegInf);
            if (a.splits == 1) {
                // A single chunk is the whole result (the merge would weigh it
                // by e^0 = 1): bf16 output and lse straight from here.
                uint32_t pk2[DPT / 2];
#pragma unroll
                for (int i = 0; i < DPT / 2; ++i) pk2[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
                uint16_t *dsto = a.o + orow * D + dq * DPT;
                if constexpr (DPT == 8)
                    *reinterpret_cast<u32x4_t *>(dsto) = u32x4_t{pk2[0], pk2[1], pk2[2], pk2[3]};
                else
                    *reinterpret_cast<u32x2_t *>(dsto) = u32x2_t{pk2[0], pk2[1]};
                if (dq == 0 && a.lse != nullptr) a.lse[((size_t)b * a.Hq + hq) * T + tq] = lse;
            } else {
                const size_t row = orow * a.splits + split;
                float *dst = a.part_o + row * D + dq * DPT;
#pragma unroll
                for (int i = 0; i < DPT; i += 4)
                    *reinterpret_cast<f32x4_t *>(dst + i) = f32x4_t{o[i], o[i + 1], o[i + 2], o[i + 3]};
                if (dq == 0) a.part_lse[row] = lse;
            }
        }
    }
    }   // items
}


// W waves per (sequence, token, query head) row, kWaves / W rows per
// workgroup.  Lane l owns d = EPL l .. EPL l + EPL - 1 of the row (EPL =
// D / 64) and the weights of splits l, l + 64, ... (0 past the last split);
// max and sum come from wave reductions (every wave of a row forms them),
// and the accumulation reads each split's weight from its lane with
// v_readlane.  Wave p of a row takes splits p, p + W, p + 2 W, ..., BLK at a
// time (the first BLK before the weights are known); indices past the last
// split are clamped to it and weighted 0, so every load is unconditional.
// With W = 1 the merge needs no LDS and no barrier; with W > 1 (few rows,
// many splits) the row's waves add their sums through LDS.
template <int D, int BLK, int W>
__global__ void __launch_bounds__(kThreads) decode_combine_kernel(DecodeArgs a)
{
    static_assert(D == 64 || D == 128, "one or two output elements per lane");
    static_assert(ATTN_MAX_SPLITS <= 256, "four split log-sum-exps per lane");
    static_assert(kWaves % W == 0 && 64 % (W * BLK) == 0, "a block's splits share one weight register");
    constexpr int EPL = D / 64;
    using vec = typename std::conditional<EPL == 2, f32x2_t, float>::type;
    constexpr int STRIDE = D / EPL;                                   // one split row, in vec units

    const int wave = (int)uniform_u32(threadIdx.x >> 6);
    const int rows = a.B * a.T * a.Hq;
    const int row_raw = blockIdx.x * (kWaves / W) + wave / W;       // (b * T + t) * Hq + hq
    if (W == 1 && row_raw >= rows) return;                           // whole waves, no barrier below
    const bool live = row_raw < rows;
    const int row = min(row_raw, rows - 1);
    const int part = wave % W;
    const int lane = threadIdx.x & 63;
    const int S = a.splits;
    const float *plse = a.part_lse + (size_t)row * S;
    const vec *po = reinterpret_cast<const vec *>(a.part_o + (size_t)row * S * D + EPL * lane);

    vec v[BLK];
#pragma unroll
    for (int u = 0; u < BLK; ++u) v[u] = po[(size_t)min(part + W * u, S - 1) * STRIDE];

    float M = kNegInf;
    bool nan = false;
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int sp = lane + 64 * j;
        x[j] = sp < S ? plse[sp] : kNegInf;
        nan |= (x[j] != x[j]);
        M = fmaxf(M, x[j]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    nan = wave_any(nan);
    float w[4];
    float wsum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w[j] = (M == kNegInf || x[j] == kNegInf) ? 0.f : exp2_fast((x[j] - M) * kLog2e);
        wsum += w[j];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);

    vec acc{};
    for (int base = 0;;) {
        const int j = base >> 6;
        const float wj = j == 0 ? w[0] : j == 1 ? w[1] : j == 2 ? w[2] : w[3];
#pragma unroll
        for (int u = 0; u < BLK; ++u)
            acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), (base & 63) + part + W * u)) * v[u];
        base += W * BLK;
        if (base >= S) break;
#pragma unroll
        for (int u = 0; u < BLK; ++u) v[u] = po[(size_t)min(base + part + W * u, S - 1) * STRIDE];
    }
    if constexpr (W > 1) {
        __shared__ vec red[kWaves][64];
        red[wave][lane] = acc;
        __syncthreads();
        if (part != 0) return;
#pragma unroll
        for (int p = 1; p < W; ++p) acc += red[wave + p][lane];
    }
    if (!live) return;

    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    if constexpr (EPL == 2) {
        const float o0 = nan ? __builtin_nanf("") : acc[0] * inv;
        const float o1 = nan ? __builtin_nanf("") : acc[1] * inv;
        reinterpret_cast<uint32_t *>(a.o + (size_t)row * D)[lane] = pack_bf16x2(o0, o1);
    } else {
        const float o0 = nan ? __builtin_nanf("") : acc * inv;
        a.o[(size_t)row * D + lane] = (uint16_t)(pack_bf16x2(o0, 0.f) & 0xffffu);
    }
    if (a.lse != nullptr && lane == 0) {
        const int th = row % (a.T * a.Hq);     // lse is [B, Hq, T]
        const size_t li = ((size_t)(row / (a.T * a.Hq)) * a.Hq + th % a.Hq) * a.T + th / a.Hq;
        a.lse[li] = nan ? __builtin_nanf("") : (wsum > 0.f ? M + logf(wsum) : kNegInf);
    }
}

// Up to eight splits: D / 4 lanes per row (4 consecutive d each, so two
// rows per wave at D = 128), every lane loading its row's few log-sum-exps
// itself (the lanes of a row read the same addresses) and forming max,
// weights and sum with no cross-lane step.  All loads are issued at once,
// indices past the last split clamped to it and weighted 0.
template <int D, int SMAX>
__global__ void __launch_bounds__(kThreads) decode_combine_small_kernel(DecodeArgs a)
{
    static_assert(D == 64 || D == 128, "16 or 32 lanes per row");
    constexpr int LPR = D / 4;
    const int rows = a.B * a.T * a.Hq;
    const int row = (int)((blockIdx.x * (unsigned)kThreads + threadIdx.x) / LPR);   // (b * T + t) * Hq + hq
    if (row >= rows) return;                                         // no cross-lane steps below
    const int c = threadIdx.x % LPR;
    const int S = a.splits;
    const float *plse = a.part_lse + (size_t)row * S;
    const f32x4_t *po = reinterpret_cast<const f32x4_t *>(a.part_o + (size_t)row * S * D) + c;

    f32x4_t v[SMAX];
    float x[SMAX];
#pragma unroll
    for (int u = 0; u < SMAX; ++u) {
        const int sp = min(u, S - 1);
        v[u] = po[(size_t)sp * LPR];
        x[u] = plse[sp];
    }
    float M = kNegInf;
    bool nan = false;
#pragma unroll
    for (int u = 0; u < SMAX; ++u)
        if (u < S) {
            nan |= (x[u] != x[u]);
            M = fmaxf(M, x[u]);
        }
    float wsum = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < SMAX; ++u) {
        const float wv = (u < S && M != kNegInf && x[u] != kNegInf) ? exp2_fast((x[u] - M) * kLog2e) : 0.f;
        wsum += wv;
        acc += wv * v[u];
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    f32x4_t o = acc * inv;
    if (nan) o = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    const u32x2_t packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    *reinterpret_cast<u32x2_t *>(a.o + (size_t)row * D + 4 * c) = packed;
    if (a.lse != nullptr && c == 0) {
        const int th = row % (a.T * a.Hq);     // lse is [B, Hq, T]
        const size_t li = ((size_t)(row / (a.T * a.Hq)) * a.Hq + th % a.Hq) * a.T + th / a.Hq;
        a.lse[li] = nan ? __builtin_nanf("") : (wsum > 0.f ? M + logf(wsum) : kNegInf);
    }
}

// Up to eight splits: the kernel above.  More: W waves per row, enough
// waves in flight for the latency of the split loads (about sixteen per
// compute unit), never more than one per eight splits, each loading all of
// its splits at once up to 16.
template <int D>
void launch_combine(const DecodeArgs &a, hipStream_t s)
{
    const long long rows = (long long)a.B * a.T * a.Hq;
    if (a.splits <= 8) {
        const dim3 grid((unsigned)((rows * (D / 4) + kThreads - 1) / kThreads)), block(kThreads);
        if (a.splits <= 2) hipLaunchKernelGGL((decode_combine_small_kernel<D, 2>), grid, block, 0, s, a);
        else if (a.splits <= 4) hipLaunchKernelGGL((decode_combine_small_kernel<D, 4>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((decode_combine_small_kernel<D, 8>), grid, block, 0, s, a);
        return;
    }
    const long long target = 16LL * compute_units();
    int W = rows >= target ? 1 : (2 * rows >= target ? 2 : 4);
    while (W > 1 && a.splits < 8 * W) W >>= 1;
    const int per_wave = (a.splits + W - 1) / W;
    const dim3 grid((unsigned)((rows * W + kWaves - 1) / kWaves)), block(kThreads);
    if (W == 4) {
        if (per_wave <= 8) hipLaunchKernelGGL((decode_combine_kernel<D, 8, 4>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((decode_combine_kernel<D, 16, 4>), grid, block, 0, s, a);
    } else if (W == 2) {
        if (per_wave <= 8) hipLaunchKernelGGL((decode_combine_kernel<D, 8, 2>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((decode_combine_kernel<D, 16, 2>), grid, block, 0, s, a);
    } else {
        hipLaunchKernelGGL((decode_combine_kernel<D, 16, 1>), grid, block, 0, s, a);
    }
}

// Dynamic LDS (unused by the kernel) that sets how many workgroups share a
// CU.  32 KiB brings the bf16, D = 128, single-tile kernel to 96 KiB, so
// that one, not two, fits a CU: on MI355X it streams 1-1.5% faster that way
// (fewer concurrent streams per CU).  8 KiB brings the e4m3, D = 128
// four-head kernel from about 50 to 58 KiB, two per CU instead of three
// (batch 64 at 16 chunks 0.436 -> 0.431 ms, other shapes unchanged).
// One-head fp8 items and several column tiles per workgroup need more
// workgroups to hide their heavier per-block work and keep their default.
template <int D, int EB, int NCT, int HPI>
constexpr unsigned occupancy_pad()
{
    if (D == 128 && EB == 2 && NCT == 1) return 32768u;
    if (D == 128 && EB == 1 && NCT == 1 && HPI > 1) return 8192u;
    return 0u;
}

// Split workgroups resident on one CU at once (queried once per kernel).
template <int D, int EB, int NCT, int HPI>
int resident_per_cu()
{
    static const int n = [] {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, reinterpret_cast<const void *>(&decode_split_kernel<D, EB, NCT, HPI>),
                                                         kThreads, occupancy_pad<D, EB, NCT, HPI>()) != hipSuccess || v <= 0)
            v = 1;
        return v;
    }();
    return n;
}

template <int D, int EB, int NCT, int HPI>
hipError_t launch_split(const DecodeArgs &a, long long n_ct, hipStream_t s)
{
    const long long units = (long long)a.B * (a.Hkv / HPI) * a.splits;
    const long long n_grp = (n_ct + NCT - 1) / NCT;
    if (units <= 0 || n_ct <= 0) return hipSuccess;
    long long grid;
    if constexpr (dynamic_items<NCT>()) {
        // As many workgroups as the GPU holds at once (never more than the
        // items), each taking items until the counter passes the last one.
        grid = std::min<long long>(units * n_grp, (long long)resident_per_cu<D, EB, NCT, HPI>() * compute_units());
    } else {
        grid = (units + 7) / 8 * 8 * n_grp;         // ids padded to whole rounds over the XCDs
    }
    constexpr unsigned pad = occupancy_pad<D, EB, NCT, HPI>();
    hipLaunchKernelGGL((decode_split_kernel<D, EB, NCT, HPI>), dim3((unsigned)grid), dim3(kThreads), pad, s, a);
    return hipGetLastError();
}

// Items of kWaves KV heads (one per wave, each wave streaming its head's
// whole chunk, items handed out longest sequence first) for single-token
// decode, when there are at least as many such items as compute units and no
// chunk is longer than 2048 tokens.  The workgroup then reads four adjacent
// head rows of each token at about the same time: a probe streams that
// pattern at 6.4 TB/s against 5.7-5.9 for one head's rows.  Measured on
// MI355X against one-head items: batch 64 at 16 chunks 0.840 -> 0.809 ms
// (bf16) and 0.448 -> 0.437 ms (e4m3), batch 4 at 128K with 64 chunks
// 0.373 -> 0.365 ms, 4 x 8192 tokens at 32 chunks 39 -> 28 us; with fewer
// items, longer chunks or several new tokens one-head items were faster
// (batch 64 at 8 chunks 0.827 against 0.842 ms; with 4 new tokens 0.845
// against 0.881-0.964 ms).
bool head_group_items(const DecodeArgs &a)
{
    if (a.T != 1 || a.Hkv % kWaves != 0) return false;
    const long long items = (long long)a.B * (a.Hkv / kWaves) * a.splits;
    const long long max_tokens = (long long)a.max_blocks * kBS;
    return items >= compute_units() && (max_tokens + a.splits - 1) / a.splits <= 2048;
}

// Column tiles per workgroup: the fewest groups of at most kMaxTiles tiles,
// the tiles spread evenly over them (the last group may run an empty tile or
// two).
template <int D, int EB>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s)
{
    const long long n_ct = ((long long)(a.Hq / a.Hkv) * a.T + 15) / 16;
    const long long n_grp = (n_ct + kMaxTiles - 1) / kMaxTiles;
    const long long nct = n_grp > 0 ? (n_ct + n_grp - 1) / n_grp : 1;
    hipError_t e;
    if (decode_wide_supported(D, EB == 1, (long long)(a.Hq / a.Hkv) * a.T)) e = launch_decode_wide(a, D, EB == 1, s);
    else if (nct <= 1) {
        e = head_group_items(a) ? launch_split<D, EB, 1, kWaves>(a, n_ct, s) : launch_split<D, EB, 1, 1>(a, n_ct, s);
    }
    else if (nct == 2) e = launch_split<D, EB, 2, 1>(a, n_ct, s);
    else if (nct == 3) e = launch_split<D, EB, 3, 1>(a, n_ct, s);
    else e = launch_split<D, EB, kMaxTiles, 1>(a, n_ct, s);
    if (n_ct <= 0 || (long long)a.B * a.Hkv * a.splits <= 0) return e;
    if (e != hipSuccess) return e;
    if (a.splits == 1) return hipSuccess;          // the split kernel wrote the result itself
    launch_combine<D>(a, s);
    return hipGetLastError();
}

}  // namespace

// Library-held decode workspace for callers that cannot allocate: one array
// per GPU the library runs on, held until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in for
// the symbol); it uses the device address that hipGetSymbolAddress returns,
// looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[ATTN_STATIC_SCRATCH_BYTES];

void *static_scratch()
{
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> ptrs[kMaxDevices];
    static std::mutex mu;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = ptrs[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = ptrs[dev].load(std::memory_order_relaxed);
    if (p != nullptr) return p;
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
    ptrs[dev].store(addr, std::memory_order_release);
    return addr;
}

hipError_t launch_decode(const DecodeArgs &a, int head_dim, bool kv_fp8, hipStream_t s)
{
    if (head_dim == 128) return kv_fp8 ? launch_d<128, 1>(a, s) : launch_d<128, 2>(a, s);
    if (head_dim == 64) return kv_fp8 ? launch_d<64, 1>(a, s) : launch_d<64, 2>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
