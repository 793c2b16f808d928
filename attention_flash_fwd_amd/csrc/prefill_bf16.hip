// prefill_bf16.hip -- exact attention forward, bf16 in/out, fp32 softmax and
// accumulation, on the gfx950 matrix cores.
//
// The FlashAttention scheme as the pages describe it ("推理加速" interview
// notes, section FlashAttention: cut Q/K/V into blocks, load blocks on chip,
// compute block attention there, online softmax, write back only the final
// output; chenyy20.com "抱infra脚", Flash Attention 基本原理 / 核心技术:
// tiling, online softmax, fusion of QK + softmax + PV; "GPU Kernel 调度：
// 大模型推理的拐点 2026", FlashAttention evolution: query blocks in parallel,
// K/V blocks pipelined, row-max / row-sum reductions; its note on the cost
// of warp specialisation motivates the two wave groups below):
//
//   one work item = 256 query rows sharing one K/V stream: 256 rows of one
//   (batch, query head), or, with causal masking, 128 rows of two or 64
//   rows of four query heads of the same KV head (as the group size
//   allows).  One workgroup per CU, 8 waves of 32 rows, takes items one
//   after another and stages its output rows through LDS so that they are
//   stored as whole rows.  Waves w and w + 4 share a SIMD; waves 0-3
//   (group 0) and 4-7 (group 1) run half a step apart, so that while one
//   wave of a SIMD works on the matrix cores the other mostly works on the
//   vector ALU.  K/V tiles of 64 keys stream through LDS (two slots each for
//   K and V) by buffer loads that write LDS directly (no register staging;
//   rows past the end of the keys read as zero).  One K/V tile load serves
//   all 256 rows, half the load traffic of 128-row workgroups.
//
//   Step s (one workgroup barrier per step):
//     matrix part   O^T += V^T P^T for tile s-1, then S^T = K Q^T for tile s
//                   (32x32x16 bf16 MFMAs; one lane = one query row; V^T from
//                   ds_read_b64_tr_b16).  The LDS reads run ahead of the
//                   products, and this part runs at raised wave priority.
//     softmax part  of tile s: mask (only tiles crossing the diagonal or the
//                   end of the keys), P = 2^(s c - m): one FMA + one v_exp_f32
//                   per score, rounded to bf16 (RNE) in the layout of the PV
//                   operand; the row sum adds the fp32 P, so lse keeps fp32
//                   accuracy.  The exponent reference m is rescaled lazily: it
//                   only has to keep every P at most 2^8, and as long as each
//                   lane's tile sum stays within 2^8 the tile needs no row max
//                   at all.  Only a row's first tile, or a tile whose scores
//                   grew past that bound, takes the row max (in-lane plus one
//                   exchange of the wave halves), rescales O and l, and forms
//                   P again.
//     group 0 runs [matrix(s), softmax(s)], group 1 [softmax(s-1), matrix(s)];
//     every wave issues its share of the loads of K(s+1) and V(s), which land
//     by the step's closing barrier.
//   A wave computes the tiles up to its own last visible key; for the
//   remaining steps of its item (past its diagonal) it only issues its
//   share of the loads.  These are separate loops, so no branch inside a
//   step ever touches the output accumulators.
//   Epilogue: O = O / l rounded to bf16, lse = (m + log2 l) * ln 2.
//
// LDS tiles are row-major with 16-byte chunks XOR-swizzled per row so that
// both the K row reads and the transposing V reads spread over all banks.
//
// Paged keys and values (chunked prefill, "抱infra脚" Paged Attention and
// Chunked Prefill): the 64 keys of a tile are 4 cache blocks of 16 tokens;
// wave w loads its 8 rows of block 4 j + w / 2, whose physical id comes
// through the scalar cache one step ahead.
//
// Work items: one per (q-tile, query head, batch).  Item ids are mapped so
// that all query heads of one (batch, KV head) belong to the same XCD (ids
// go round-robin over the 8 XCDs), each XCD works through its (batch, KV
// head) pairs one at a time, and within a pair the longest causal q-tiles
// come first: the pair's K/V stays in that XCD's L2.  The grid is
// persistent: one workgroup per CU, each looping over items of its XCD, so
// that a CU goes from one item to the next without waiting for a workgroup
// to retire and another to be dispatched.
#include <algorithm>
#include <type_traits>

#include "gfx950.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBR = 256;      // query rows per work item (all heads of the item together)
constexpr int kBC = 64;       // keys per K/V tile
constexpr int kBS = 16;       // tokens per cache block (paged keys and values)
constexpr int kThreads = 512;
constexpr int kWaves = 8;

// An empty volatile asm statement: placed inside a rarely taken branch it
// keeps the compiler from turning the branch into unconditional arithmetic.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Instruction-class masks of the scheduling-group builtin.
constexpr int kSchedMfma = 0x008, kSchedVmem = 0x010, kSchedDsRead = 0x100;
#define SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

template <int D>
struct Tile {
    static constexpr int cpr = D / 8;                     // 16-byte chunks per row
    static constexpr int elems = kBC * D;                 // bf16 elements per K or V tile
    static constexpr int lpw = kBC * cpr / 64 / kWaves;   // 1 KiB LDS-direct loads per wave per K or V tile
    // Physical chunk of logical chunk c in row r.
    static __device__ __forceinline__ int swz(int r, int c)
    {
        if constexpr (D == 128)
            return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
        else
            return c ^ ((r >> 1) & 7);
    }
};

// Item L -> (batch b, first query head hq, q-tile qt); an item covers hpi
// consecutive query heads of one KV group.
__device__ __forceinline__ void map_workgroup(int L, const PrefillArgs &a, int n_qtiles, int hpi,
                                              int &b, int &hq, int &qt)
{
    const int G = a.Hq / a.Hkv / hpi;               // items per (q-tile, KV head)
    const int groups = a.B * a.Hkv;                 // (batch, KV head) pairs
    int qt_rev, g, hg;
    if (groups % 8 == 0) {
        const int xcd = L & 7, r = L >> 3;
        // group-major on each XCD: all q-tiles of one (batch, KV head) pair,
        // heaviest first, before the next pair, so that one pair's K/V is
        // the XCD's L2 working set
        const int per = n_qtiles * G;               // items of one pair
        const int gi = r / per;
        const int rem = r - gi * per;
        qt_rev = rem / G;
        hg = rem % G;
        g = xcd + 8 * gi;
    } else {
        const int per = groups * G;
        qt_rev = L / per;
        const int rem = L - qt_rev * per;
        g = rem / G;
        hg = rem % G;
    }
    b = g / a.Hkv;
    hq = ((g % a.Hkv) * G + hg) * hpi;
    qt = n_qtiles - 1 - qt_rev;
}

// HPI query heads of one KV group per item, 256 / HPI rows each.  The K/V
// tiles still serve 256 rows, but the causal diagonal of an item crosses
// 4 / HPI tiles, so fewer waves sit idle while the others finish their
// diagonal tiles (with HPI = 4, none).
template <int D, bool CAUSAL, bool PAGED, int HPI>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_kernel(PrefillArgs a, int n_qtiles, int n_items)
{
    static_assert(HPI == 1 || HPI == 2 || HPI == 4, "heads per item");
    constexpr int RPH = kBR / HPI;                  // rows per head of an item
    using T = Tile<D>;
    // Distinct arrays per slot, so that the compiler's wait for a slot's
    // LDS-direct loads never covers the loads in flight to the other slot.
    __shared__ __attribute__((aligned(1024))) uint16_t k_s0[T::elems];
    __shared__ __attribute__((aligned(1024))) uint16_t k_s1[T::elems];
    __shared__ __attribute__((aligned(1024))) uint16_t v_s0[T::elems];
    __shared__ __attribute__((aligned(1024))) uint16_t v_s1[T::elems];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2;
    const int l32 = lane & 31, h = lane >> 5;

    // Workgroup w stays on XCD w % 8 and takes that XCD's items (ids L with
    // L % 8 == w % 8) in rounds of one item per workgroup, the direction
    // alternating between rounds: with the heaviest causal q-tiles first,
    // every workgroup then gets about the same number of tiles.  Only the
    // last round can run out of items, so the first missing item ends the
    // loop.
    const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3, nk = gridDim.x >> 3;
    const int per_xcd = (n_items + 7) >> 3;
    for (int round = 0;; ++round) {
    const int rr = round * nk + ((round & 1) ? nk - 1 - kx : kx);
    const int item = rr * 8 + xcd;
    if (rr >= per_xcd || item >= n_items) break;

    int b, hq0, qt;
    map_workgroup(item, a, n_qtiles, HPI, b, hq0, qt);
    const int G = a.Hq / a.Hkv, hk = hq0 / G;
    // This wave's head and 32-row block.  HPI = 2: waves 0-3 take rows
    // 0..127 of head hq0 and waves 4-7 rows 127..0 of head hq0 + 1, so the
    // two waves of a SIMD (w and w + 4) reach the diagonal at different
    // tiles.  HPI = 4: waves 2j and 2j + 1 take rows 0..63 of head hq0 + j.
    const int hq = hq0 + (HPI == 4 ? (wave >> 1) : HPI == 2 ? (wave >> 2) : 0);
    const int rb = HPI == 4 ? (wave & 1) : HPI == 2 ? ((wave < 4) ? wave : 7 - wave) : wave;
    const int i0 = qt * RPH;
    const int q0 = i0 + rb * 32;        // first query row of this wave (uniform)
    const int my_q = q0 + l32;          // query row of this lane
    // Keys of this sequence.  Paged: read through the scalar cache (so that
    // everything derived from it stays wave-uniform); a length outside the
    // table's reach marks the sequence bad (NaN output) and reads no key.
    int Sk = a.Sk;
    bool bad = false;
    if constexpr (PAGED) {
        Sk = ((const int32_t __attribute__((address_space(4))) *)a.ctx_lens)[b];
        if (Sk < 0 || Sk > a.max_blocks * kBS) {
            bad = true;
            Sk = 0;
        }
    }
    const int diag = Sk - a.Sq;         // key j visible to row i iff j <= i + diag

    int kend = Sk;                      // keys [0, kend) may be visible to this item
    if (CAUSAL) kend = min(Sk, min(a.Sq, i0 + RPH) + diag);
    const int n = kend > 0 ? (kend + kBC - 1) / kBC : 0;
    // Tiles [0, nw) hold keys visible to some row of this wave; from step nw
    // on the wave only issues its share of the loads (its P would be 0).
    int kend_w = Sk;
    if (CAUSAL) kend_w = min(Sk, min(a.Sq, q0 + 32) + diag);
    if (q0 >= a.Sq) kend_w = 0;
    const int nw = kend_w > 0 ? (kend_w + kBC - 1) / kBC : 0;
    // Tiles before first_masked are fully visible to every row of this wave.
    int first_masked = Sk / kBC;
    if (CAUSAL) first_masked = min(first_masked, max(0, (q0 + diag + 1) / kBC));

    // Exponent scale c = scale * log2(e), made non-negative by flipping the
    // sign of Q (exact in bf16) when the caller's scale is negative, and at
    // least FLT_MIN: a masked score (-inf) then always maps to 2^-inf = 0,
    // and a zero scale still gives uniform weights.
    const bool neg = a.scale_log2 < 0.f;
    const float c = fmaxf(neg ? -a.scale_log2 : a.scale_log2, 1.17549435e-38f);

    // Q^T operand of S^T = K Q^T: lane (h, l32) holds q[my_q][16ks + 8h .. +8].
    u32x4_t qf[D / 16];
    {
        const uint16_t *qg = static_cast<const uint16_t *>(a.q);
        const size_t row = ((size_t)b * a.Sq + min(my_q, a.Sq - 1)) * a.Hq + hq;
        const uint16_t *qp = qg + row * D + 8 * h;
        const uint32_t flip = neg ? 0x80008000u : 0u;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            u32x4_t x = *reinterpret_cast<const u32x4_t *>(qp + 16 * ks);
            x ^= flip;
            qf[ks] = my_q < a.Sq ? x : u32x4_t{0, 0, 0, 0};
        }
    }

    // ---- K/V streaming: buffer loads that write LDS directly ------------
    const uint32_t row_bytes = (uint32_t)(a.Hkv * D * 2);
    // Per-lane source offsets (bytes) of the 16-byte chunks this lane's loads
    // deliver: load i of wave w fills LDS chunk slots (w * lpw + i) * 64 + lane,
    // rows 8 w .. 8 w + 7 of the tile.  Contiguous: relative to the tile's
    // first key; paged: relative to the first token of cache block w / 2.
    uint32_t src_off[T::lpw];
#pragma unroll
    for (int i = 0; i < T::lpw; ++i) {
        const int slot = (wave * T::lpw + i) * 64 + lane;
        const int r = slot / T::cpr, p = slot % T::cpr;
        src_off[i] = (uint32_t)(PAGED ? r - kBS * (wave >> 1) : r) * row_bytes + (uint32_t)T::swz(r, p) * 16u;
    }
    // Loads of one K or V tile; off (wave-uniform) is added to every lane's
    // source offset.
    auto load_slot = [&](__amdgpu_buffer_rsrc_t r, uint16_t *dst, uint32_t off) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < T::lpw; ++i) buffer_load_lds16(r, dst + (wave * T::lpw + i) * 64 * 8, src_off[i] + off);
    };

    // Contiguous keys: one descriptor each for K and V over this (batch, KV
    // head)'s keys, made once per item; tile j starts tile_off(j) bytes in.
    // Rows past the keys, and tiles past the item's last one (offset span),
    // read as zero.
    const size_t head_off = PAGED ? 0 : ((size_t)b * a.Sk * a.Hkv + hk) * D;      // elements
    const char *kbase = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.k) + head_off);
    const char *vbase = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.v) + head_off);
    const uint32_t span = Sk > 0 ? (uint32_t)(((size_t)(Sk - 1) * a.Hkv * D + D) * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, span), rv = make_rsrc(vbase, span);
    const int n_u = (int)uniform_u32((uint32_t)n);
    const uint32_t span_u = uniform_u32(span), row_bytes_u = uniform_u32(row_bytes);
    auto tile_off = [&](int j) __attribute__((always_inline)) {
        return j < n_u ? (uint32_t)(j * kBC) * row_bytes_u : span_u;
    };

    // Paged keys: wave w's cache block of tile t is 4 t + w / 2; its physical
    // id is looked up one step ahead through the scalar cache.
    const int n_lblocks = (Sk + kBS - 1) / kBS;
    const int32_t __attribute__((address_space(4))) *tb =
        (const int32_t __attribute__((address_space(4))) *)(a.block_table + (PAGED ? (size_t)b * a.max_blocks : 0));
    const uint32_t blk_bytes = (uint32_t)kBS * row_bytes;
    // Rows of tile t that this wave's block holds (0 past the keys or past
    // the workgroup's tiles).
    auto block_rows = [&](int t) __attribute__((always_inline)) {
        const int lb = (kBC / kBS) * t + (wave >> 1);
        return ((t < n) & (lb < n_lblocks)) ? min(kBS, Sk - kBS * lb) : 0;
    };
    // Physical id of this wave's block of tile t, read through the scalar
    // cache at an index clamped into the table row (the value only matters
    // when the block holds rows).
    auto lookup = [&](int t) __attribute__((always_inline)) {
        return (PAGED && a.max_blocks > 0) ? tb[min((kBC / kBS) * t + (wave >> 1), a.max_blocks - 1)] : 0;
    };
    // Descriptor of this wave's block of tile t with physical id p; an id
    // outside the pool marks the sequence bad and reads nothing.
    auto rsrc_block = [&](const void *cache, int t, int p) __attribute__((always_inline)) {
        const int rows = block_rows(t);
        // bitwise, not short-circuit, logic: straight-line scalar code
        const bool wrong = (rows > 0) & ((p < 0) | (p >= a.num_blocks));
        bad = bad | wrong;
        const bool use = (rows > 0) & !wrong;
        const size_t off = use ? (size_t)(uint32_t)p * blk_bytes + (size_t)hk * D * 2 : 0;
        const uint32_t num = use ? (uint32_t)(rows - 1) * row_bytes + D * 2 : 0u;
        return make_rsrc(static_cast<const char *>(cache) + off, num);
    };
    // Step s loads K(s+1) and V(s) through descriptors made at the end of the
    // previous step (scalar work kept out of the matrix part); the block ids
    // are read one step before the descriptors need them.
    int id_a = lookup(1), id_b = lookup(2);          // tiles s + 1 and s + 2 at step s
    __amdgpu_buffer_rsrc_t desc_k = rsrc_block(a.k, 1, id_a), desc_v = rsrc_block(a.v, 0, lookup(0));
    auto advance = [&](int s) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            desc_v = rsrc_block(a.v, s + 1, id_a);
            desc_k = rsrc_block(a.k, s + 2, id_b);
            id_a = id_b;
            id_b = lookup(s + 3);
        }
    };

    // ---- per-lane LDS read offsets (elements) ----------------------------
    // K operand (S^T A operand): row l32 (+32 kb), chunk 2 kk + h.
    int k_rd[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) k_rd[kk] = l32 * D + T::swz(l32, 2 * kk + h) * 8;
    // V^T operand via transpose reads: within 16-lane group (hh, dh), source
    // lane s points at key row 4 hh + 8 t + s/4 and d = 32 db + 16 dh + 4 (s % 4).
    const int s16 = lane & 15, g16 = lane >> 4, hh = g16 >> 1, dh = g16 & 1;
    int v_rd[2][D / 32];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int r = 4 * hh + 8 * t + (s16 >> 2);
            const int d = 32 * db + 16 * dh + 4 * (s16 & 3);
            v_rd[t][db] = r * D + T::swz(r, d >> 3) * 8 + (d & 7);
        }

    // ---- per-lane softmax state and accumulators --------------------------
    f32x16_t oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m = kNegInf;      // exponent reference (log2 domain) of this row
    float lsum = 0.f;       // this lane's share of the row sum
    const f32x16_t zero16 = {};
    f32x16_t sc[2];          // S^T of a tile between its QK and its softmax
    u32x4_t pk[2][2];        // P of a tile between its softmax and its PV

    constexpr int NMF = D / 8;                 // MFMAs per tile and wave, for QK and for PV
    constexpr int PVA = 4, QKA = 4;            // products the LDS reads run ahead

    auto read_v = [&](const uint16_t *vs, u32x4_t (&vf)[2][2][D / 32]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const int e = (32 * kb + 16 * cc) * D;
                    const u32x2_t lo = lds_read_tr16(vs + v_rd[0][db] + e);
                    const u32x2_t hi = lds_read_tr16(vs + v_rd[1][db] + e);
                    vf[kb][cc][db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
                }
    };
    auto read_k = [&](const uint16_t *ks, u32x4_t (&kf)[D / 16][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) kf[kk][kb] = *reinterpret_cast<const u32x4_t *>(ks + k_rd[kk] + 32 * kb * D);
    };
    // O^T += V^T P^T; the S^T accumulator layout is the B operand once the
    // keys of each MFMA are taken in the accumulator's order.
    auto pv = [&](const u32x4_t (&vf)[2][2][D / 32]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) oacc[db] = mfma_32x32x16_bf16(vf[kb][cc][db], pk[kb][cc], oacc[db]);
    };
    // S^T = K Q^T, both 32-key halves of the tile.
    auto qk = [&](const u32x4_t (&kf)[D / 16][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sc[kb] = mfma_32x32x16_bf16(kf[kk][kb], qf[kk], kk == 0 ? zero16 : sc[kb]);
    };

    // Matrix part of a steady step: PV of the previous tile, then QK of this
    // one; a single code path (no branch touches the accumulators).
    auto mma_full = [&](const uint16_t *ks, const uint16_t *vs, auto &&issue) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        u32x4_t vf[2][2][D / 32];
        u32x4_t kf[D / 16][2];
        read_v(vs, vf);
        read_k(ks, kf);
        issue();
        pv(vf);
        qk(kf);
        SCHED_GROUP(kSchedDsRead, 2 * PVA);
        SCHED_GROUP(kSchedVmem, 4 * T::lpw);
#pragma unroll
        for (int i = 0; i < NMF - PVA; ++i) {
            SCHED_GROUP(kSchedMfma, 1);
            SCHED_GROUP(kSchedDsRead, 2);
        }
#pragma unroll
        for (int i = 0; i < PVA; ++i) {
            SCHED_GROUP(kSchedMfma, 1);
            if (i < QKA) SCHED_GROUP(kSchedDsRead, 1);
        }
#pragma unroll
        for (int i = 0; i < NMF - QKA; ++i) {
            SCHED_GROUP(kSchedMfma, 1);
            SCHED_GROUP(kSchedDsRead, 1);
        }
        SCHED_GROUP(kSchedMfma, QKA);
        __builtin_amdgcn_s_setprio(0);
    };
    auto mma_qk_only = [&](const uint16_t *ks, auto &&issue) __attribute__((always_inline)) {
        u32x4_t kf[D / 16][2];
        read_k(ks, kf);
        issue();
        qk(kf);
    };
    auto mma_pv_only = [&](const uint16_t *vs) __attribute__((always_inline)) {
        u32x4_t vf[2][2][D / 32];
        read_v(vs, vf);
        pv(vf);
    };

    // Softmax of tile s.
    auto softmax = [&](int s) __attribute__((always_inline)) {
        if (s >= first_masked) {
            keep_branch();
            // last visible key offset in the tile, less this lane's 4 h, so that
            // every compare is against an inline constant
            const int lim = (CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1) - s * kBC - 4 * h;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int ko = 32 * kb + 8 * (v >> 2) + (v & 3);
                    sc[kb][v] = ko <= lim ? sc[kb][v] : kNegInf;
                }
        }
        // P = 2^(s c - m) -> bf16 pairs; returns this lane's sum of the fp32
        // values (the row sum keeps fp32 accuracy).
        auto exp_tile = [&](float nm) __attribute__((always_inline)) {
            float t = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float p0 = exp2_fast(__builtin_fmaf(sc[kb][8 * cc + 2 * e], c, nm));
                        const float p1 = exp2_fast(__builtin_fmaf(sc[kb][8 * cc + 2 * e + 1], c, nm));
                        pk[kb][cc][e] = pack_bf16x2(p0, p1);
                        t = (kb | cc | e) ? t + (p0 + p1) : p0 + p1;
                    }
            return t;
        };
        // The reference m only has to bound the exponents: every P must stay
        // at most 2^8.  Once every row of the wave has a finite m, the tile's
        // P are formed against it first; a lane sum of at most 2^8 shows that
        // no P of the lane exceeds it, and the tile is done without a row max.
        // Otherwise (a row's first visible keys, or scores that grew past
        // the reference) the row max is taken and m moves to it.
        bool redo = true;
        float t = 0.f;
        if (!wave_any(m == kNegInf)) {
            t = exp_tile(-m);
            redo = wave_any(t > 256.0f);
        }
        if (redo) {
            keep_branch();
            // Row max of the raw scores (c > 0, so scaling preserves order),
            // as four independent partial maxima.
            float mp[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mp[2 * kb + (v >> 3)] = fmaxf(mp[2 * kb + (v >> 3)], sc[kb][v]);
            float mraw = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
            mraw = pair_max_halves(mraw);
            const float mx = mraw == kNegInf ? kNegInf : mraw * c;
            const float m_new = fmaxf(m, mx);
            const bool grow = m_new > m;
            if (wave_any(grow)) {
                const float alpha = grow ? exp2_fast(m - m_new) : 1.0f;
                m = grow ? m_new : m;
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
            }
            t = exp_tile((m == kNegInf) ? 0.f : -m);
        }
        lsum += t;
    };

    // ---- steps s = 0..n: K(s) in k_s[s & 1], V(s) in v_s[s & 1] ----------
    // Step s loads K(s+1) and V(s) (slots freed by the previous step's
    // barrier); they land by step s's closing barrier.
    auto issue = [&](int s, uint16_t *k_ld, uint16_t *v_ld) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            load_slot(desc_k, k_ld, 0u);
            load_slot(desc_v, v_ld, 0u);
        } else {
            load_slot(rk, k_ld, tile_off(s + 1));
            load_slot(rv, v_ld, tile_off(s));
        }
    };
    if constexpr (PAGED)
        load_slot(rsrc_block(a.k, 0, lookup(0)), k_s0, 0u);
    else
        load_slot(rk, k_s0, tile_off(0));
    __syncthreads();
    if (n > 0) {
        auto body0 = [&](int s, const uint16_t *ks, const uint16_t *vs, uint16_t *k_ld, uint16_t *v_ld)
            __attribute__((always_inline)) {
            mma_full(ks, vs, [&]() __attribute__((always_inline)) { issue(s, k_ld, v_ld); });
            softmax(s);
            advance(s);
            __syncthreads();
        };
        auto body1 = [&](int s, const uint16_t *ks, const uint16_t *vs, uint16_t *k_ld, uint16_t *v_ld)
            __attribute__((always_inline)) {
            issue(s, k_ld, v_ld);
            softmax(s - 1);
            mma_full(ks, vs, []() {});
            advance(s);
            __syncthreads();
        };
        // A step that only issues this wave's loads.
        auto idle = [&](int s) __attribute__((always_inline)) {
            if (s & 1)
                issue(s, k_s0, v_s1);
            else
                issue(s, k_s1, v_s0);
            advance(s);
            __syncthreads();
        };
        const int m_end = min(nw, n);     // steps [1, m_end) run in full
        if (grp == 0) {
            mma_qk_only(k_s0, [&]() __attribute__((always_inline)) { issue(0, k_s1, v_s0); });
            softmax(0);
            advance(0);
            __syncthreads();
            int s = 1;
            for (; s + 1 < m_end; s += 2) {
                body0(s, k_s1, v_s0, k_s0, v_s1);
                body0(s + 1, k_s0, v_s1, k_s1, v_s0);
            }
            if (s < m_end) body0(s++, k_s1, v_s0, k_s0, v_s1);
            if (s == nw && s < n) {
                // this wave's last PV (tile nw - 1), then loads only
                if (s & 1) {
                    mma_pv_only(v_s0);
                    issue(s, k_s0, v_s1);
                } else {
                    mma_pv_only(v_s1);
                    issue(s, k_s1, v_s0);
                }
                advance(s);
                __syncthreads();
                ++s;
            }
            for (; s < n; ++s) idle(s);
            if (nw >= n) mma_pv_only((n & 1) ? v_s0 : v_s1);
            __syncthreads();
        } else {
            issue(0, k_s1, v_s0);
            mma_qk_only(k_s0, []() {});
            advance(0);
            __syncthreads();
            int s = 1;
            for (; s + 1 < m_end; s += 2) {
                body1(s, k_s1, v_s0, k_s0, v_s1);
                body1(s + 1, k_s0, v_s1, k_s1, v_s0);
            }
            if (s < m_end) body1(s++, k_s1, v_s0, k_s0, v_s1);
            if (s == nw && s < n) {
                if (s & 1)
                    issue(s, k_s0, v_s1);
                else
                    issue(s, k_s1, v_s0);
                softmax(s - 1);
                mma_pv_only((s & 1) ? v_s0 : v_s1);
                advance(s);
                __syncthreads();
                ++s;
            }
            for (; s < n; ++s) idle(s);
            if (nw >= n) {
                softmax(n - 1);
                mma_pv_only((n & 1) ? v_s0 : v_s1);
            }
            __syncthreads();
        }
    }

    // ---- epilogue ----------------------------------------------------------
    if constexpr (PAGED) bad = __syncthreads_or(bad);
    const float ltot = pair_sum_halves(lsum);
    {
        // O rows through LDS, so that the stores write whole rows: each wave
        // puts its 32 rows (bf16, 16-byte chunks XOR-swizzled by row) in its
        // own 32 x D slice of the idle K/V ring (free since the last step's
        // barrier), then 16 lanes (D = 128) or 8 (D = 64) store one row.
        // Rows past the queries fall outside the store descriptor.
        constexpr int CPR = D / 8;                  // 16-byte chunks per row
        float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
        if (PAGED && bad) inv = __builtin_nanf("");
        uint16_t *stage = (wave < 2 ? k_s0 : wave < 4 ? k_s1 : wave < 6 ? v_s0 : v_s1) + (wave & 1) * 32 * D;
        // Lane index through opaque(): the addresses below are then formed
        // here, not hoisted out of the item loop into registers held
        // across the main loop.
        const int ln = opaque(lane), r32 = ln & 31, hh = ln >> 5;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                // d = 32 db + 8 g4 + 4 h .. +3: half h of chunk 4 db + g4 of row l32
                const u32x2_t w = {pack_bf16x2(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv),
                                   pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
                const int c = (4 * db + g4) ^ (r32 % CPR);
                *reinterpret_cast<u32x2_t *>(stage + r32 * D + 8 * c + 4 * hh) = w;
            }
        }
        const int rows = max(0, min(32, a.Sq - q0));
        const uint32_t rstride = (uint32_t)(a.Hq * D * 2);
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(static_cast<uint16_t *>(a.o) + (((size_t)b * a.Sq + q0) * a.Hq + hq) * D,
                      rows > 0 ? (uint32_t)(rows - 1) * rstride + D * 2 : 0u);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 32 * CPR / 64; ++i) {
            const int r = i * (64 / CPR) + ln / CPR, c = ln % CPR;
            const u32x4_t x = *reinterpret_cast<const u32x4_t *>(stage + r * D + 8 * (c ^ (r % CPR)));
            __builtin_amdgcn_raw_buffer_store_b128(x, ro, (uint32_t)r * rstride + 16u * c, 0, 0);
        }
    }
    if (my_q < a.Sq) {
        if (a.lse != nullptr && h == 0)
            a.lse[((size_t)b * a.Hq + hq) * a.Sq + my_q] =
                (PAGED && bad) ? __builtin_nanf("") : (ltot > 0.f ? (m + __log2f(ltot)) * kLn2 : kNegInf);
    }
    // Every wave is done with its slice of the ring before the next item's
    // K tile 0 lands there (the output stores may still be in flight).
    lds_barrier();
    }   // items
}

template <int D, bool CAUSAL, bool PAGED, int HPI>
hipError_t launch_items(const PrefillArgs &a, hipStream_t s)
{
    constexpr int RPH = kBR / HPI;
    const int n_qtiles = (a.Sq + RPH - 1) / RPH;
    const long long items = (long long)n_qtiles * (a.Hq / HPI) * a.B;
    if (items <= 0) return hipSuccess;
    // One workgroup per CU (a workgroup fills a CU's registers), a multiple
    // of 8 so that each workgroup keeps to the items of one XCD.
    const long long grid = std::min<long long>((items + 7) / 8 * 8, std::max(8, compute_units() / 8 * 8));
    hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, PAGED, HPI>), dim3((unsigned)grid), dim3(kThreads), 0, s, a,
                       n_qtiles, (int)items);
    return hipGetLastError();
}

// Causal: as many query heads per item (4, 2 or 1) as divide the heads per
// KV head.
template <int D, bool CAUSAL, bool PAGED>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s)
{
    const int G = a.Hq / a.Hkv;
    if constexpr (CAUSAL) {
        if (G % 4 == 0) return launch_items<D, CAUSAL, PAGED, 4>(a, s);
        if (G % 2 == 0) return launch_items<D, CAUSAL, PAGED, 2>(a, s);
    }
    return launch_items<D, CAUSAL, PAGED, 1>(a, s);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, bool causal, hipStream_t s)
{
    if (head_dim == 128) return causal ? launch_one<128, true, false>(a, s) : launch_one<128, false, false>(a, s);
    if (head_dim == 64) return causal ? launch_one<64, true, false>(a, s) : launch_one<64, false, false>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_paged_bf16(const PrefillArgs &a, int head_dim, bool causal, hipStream_t s)
{
    if (head_dim == 128) return causal ? launch_one<128, true, true>(a, s) : launch_one<128, false, true>(a, s);
    if (head_dim == 64) return causal ? launch_one<64, true, true>(a, s) : launch_one<64, false, true>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
