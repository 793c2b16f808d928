// decode_wide.hip -- split-KV decode over a paged KV cache (bf16, or e4m3
// at head_dim 128) for many (token, head) columns: several new tokens per sequence (the verification
// step of speculative decoding, "推理加速" interview notes, section
// speculative decoding; "GPU Kernel 调度：大模型推理的拐点 2026", paragraph
// on speculative decoding with Flash-Decoding) or large query-head groups.
// Same chunking and partials as the decode kernel in decode.hip (Flash
// Decoding, same page: chunks of the cached K/V in parallel, partial outputs
// merged by log-sum-exp), same cache layout ("抱infra脚", section Paged
// Attention).
//
// With more than 32 columns (column = new token t times G query heads of
// the KV head, plus head g), the decode kernel's 16-column tiles cost: its
// PV products use the K = 16 matrix-core form, which gfx950 runs at half
// the rate of the K = 32 forms, and more than four tiles take a second pass
// over the chunk.  Here a workgroup of NC waves owns 32 NC columns, one
// wave per 32 columns, on the 32x32x16 bf16 products for both S and PV:
//
//   step = 32 tokens (two cache blocks), shared by all NC waves through an
//   NS-slot LDS ring filled by LDS-direct buffer loads (each wave issues
//   its share; loads run NS - 1 steps ahead; one workgroup barrier a step)
//   S^T (32 tokens x 32 columns) = K Q^T      D / 16 products
//   online softmax per column (lane l: column l % 32, 16 tokens; the two
//   wave halves hold the same column), lazy rescale as in the prefill
//   kernel, P rounded to bf16 in the layout of the PV operand
//   O^T (D x 32 columns) += V^T P^T           D / 16 products
//
// e4m3 caches: K operands are widened to bf16 in registers as they are
// read; after each step's loads land, the waves widen the step's V rows
// into a shared bf16 copy in LDS (a quarter or half each) and meet at one
// more barrier, so the transposing V reads are those of the bf16 path.
//
// Each wave owns its columns for the whole chunk, so no partials are merged
// across waves: the normalised output and log-sum-exp of every column go
// straight to the partial buffers (or, with a single chunk, to the output).
//
// Items are (column group, chunk, KV head, sequence).  With one column group
// (up to 32 NC columns) as many workgroups as the GPU holds stay resident and
// take items from the work counter in the workspace, as the decode kernel in
// decode.hip does; with more, each workgroup computes one item of a grid
// laid out so that the groups of a chunk share an XCD's L2.
#include <algorithm>

#include "gfx950.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBS = 16;        // tokens per cache block
constexpr int kStep = 32;      // tokens per step: two cache blocks
constexpr int kColsPerWave = 32;
constexpr int kMaxRanked = 256;  // sequences ranked by length for the item order

template <int D, int EB = 2>
struct WideTile {
    static constexpr int row_bytes = EB * D;                 // one token row of one KV head (bf16 or e4m3)
    static constexpr int cpr = row_bytes / 16;               // 16-byte chunks per row
    static constexpr int rows_per_dma = 1024 / row_bytes;    // rows one wave-wide 16-byte load fills
    static constexpr int dmas = kStep / rows_per_dma;        // such loads per K (or V) slot
    static constexpr int slot_bytes = kStep * row_bytes;
    // LDS position of logical 16-byte chunk c of row r (an involution): the
    // row reads of K and the transposing reads of V spread over all banks.
    // Periodic in r with period 16.
    static __device__ __forceinline__ int swz(int r, int c)
    {
        if constexpr (EB == 2)
            return D == 128 ? c ^ (((r & 3) << 2) | ((r >> 2) & 3)) : c ^ ((r >> 1) & 7);
        else   // rows of 128 or 64 bytes
            return D == 128 ? c ^ ((r >> 1) & 7) : c ^ ((r >> 2) & 3);
    }
};

// Wait until at most n of this wave's vector-memory loads are outstanding
// (expcnt left unconstrained; with lds, also every LDS access of the wave).
template <int n, bool lds = false>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (lds ? 0 : (0xF << 8)));
}

// Wait for this wave's LDS accesses only (vector-memory loads stay in flight).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (0x7 << 4)); }

// Workgroup barrier that waits for nothing by itself: the caller's
// wait_vmcnt decides which loads must have landed.  (A fence-based barrier
// would wait for every LDS-direct load in flight, including those of the
// steps after the next.)  The memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void plain_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int D, int NC, int NS, bool DYN, int EB>
__global__ void __launch_bounds__(64 * NC) __attribute__((amdgpu_waves_per_eu(2)))
decode_wide_kernel(DecodeArgs a)
{
    static_assert(NS == 2 || NS == 3, "ring depth");
    using T = WideTile<D, EB>;      // the cache's rows in the ring
    using TB = WideTile<D, 2>;      // bf16 rows (V as the transposing reads see it)
    static_assert(T::dmas % NC == 0, "loads split evenly over the waves");
    constexpr int LPW = 2 * T::dmas / NC;          // this wave's loads per step (K and V)
    // One array per slot, so that the compiler's wait before a slot's reads
    // never covers loads in flight to another slot.
    __shared__ __attribute__((aligned(1024))) uint8_t k0[T::slot_bytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[T::slot_bytes];
    __shared__ __attribute__((aligned(1024))) uint8_t k1[T::slot_bytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v1[T::slot_bytes];
    // e4m3 caches: the step's V rows widened to bf16, shared by the waves.
    __shared__ __attribute__((aligned(1024))) uint8_t cv[EB == 1 ? TB::slot_bytes : 16];

    const int lane = threadIdx.x & 63;
    const int wave = (int)uniform_u32(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;

    const int G = a.Hq / a.Hkv;
    const int TQ = a.T;
    const int GT = G * TQ;
    constexpr int WG_COLS = kColsPerWave * NC;
    const int n_grp = (GT + WG_COLS - 1) / WG_COLS;
    const int units = a.B * a.Hkv * a.splits;
    // DYN (one column group): workgroup w runs item w first; later items come
    // from the counter, tickets 0, 1, ... standing for items gridDim.x,
    // gridDim.x + 1, ...  Workgroup 0 zeroes the counter as it starts.
    // Whatever the counter held before, no item is lost: a ticket taken
    // before the reset either lies past the end (that workgroup stops early)
    // or is issued again after it (the item is computed twice, with identical
    // results), and workgroup 0 keeps taking tickets until the counter passes
    // the last item.  Thread 0 takes the next ticket as an item's outputs are
    // written and hands the item to the other waves through an LDS word; the
    // barrier that ends every item orders that write after their reads.
    __shared__ unsigned item_slot[1];
    __shared__ int bad_s[NC];                       // per wave: a bad block id seen in this item
    unsigned ticket = 0;
    // DYN: items go out longest sequence first (list scheduling), so that a
    // long sequence's chunks do not start last: each workgroup ranks the
    // sequences by length (ties by index, a permutation) into an LDS table
    // as it starts.  More sequences than the table holds keep their order.
    __shared__ int16_t seq_order[DYN ? kMaxRanked : 1];
    __shared__ int ctx_s[DYN ? kMaxRanked : 1];
    const bool ranked = DYN && a.B <= kMaxRanked;
    if (ranked) {
        for (int i = threadIdx.x; i < a.B; i += 64 * NC) ctx_s[i] = a.ctx_lens[i];
        __syncthreads();
        for (int i = threadIdx.x; i < a.B; i += 64 * NC) {
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
        unsigned item = blockIdx.x;
        if (round > 0) {
            if (threadIdx.x == 0)
                item_slot[0] = ticket < (unsigned)units - gridDim.x ? gridDim.x + ticket : (unsigned)units;
            __syncthreads();
            item = uniform_u32(item_slot[0]);
        }
        if (item >= (unsigned)units) break;
        grp = 0;
        unit = (int)item;
    } else {
        // Workgroup -> (column group, chunk, KV head, sequence).  The groups
        // of one (chunk, KV head, sequence) get ids 8 apart: ids go
        // round-robin over the 8 XCDs, so they run at the same time on one
        // XCD and share its L2 copy of the chunk.
        if (round > 0) break;
        const int L = blockIdx.x, r8 = L >> 3;
        grp = r8 % n_grp;
        unit = (r8 / n_grp) * 8 + (L & 7);
        if (unit >= units) break;                   // padding of the id space (uniform)
    }
    const int split = unit % a.splits;
    const int hk = (unit / a.splits) % a.Hkv;
    const int bq = unit / (a.splits * a.Hkv);
    const int b = ranked ? (int)uniform_u32((uint32_t)seq_order[bq]) : bq;

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
    const int nsteps = (t_end - t_begin + kStep - 1) / kStep;

    // Exponent scale c = scale * log2(e), made non-negative by flipping the
    // sign of Q (exact in bf16) when the scale is negative, and at least
    // FLT_MIN, so that a masked score (-inf) always gives 2^-inf = 0.
    const bool neg = a.scale_log2 < 0.f;
    const float c = fmaxf(neg ? -a.scale_log2 : a.scale_log2, 1.17549435e-38f);

    // This lane's column: col = t G + g is query head hk G + g of new token
    // t.  Columns past G T read the last valid one with Q zeroed and are
    // never written.
    const int want = grp * WG_COLS + kColsPerWave * wave + l32;
    const bool col_ok = want < GT;
    const int col = min(want, GT - 1);
    const int tq = col / G, hq = hk * G + col % G;
    const int lim = ctx - TQ + tq;                  // last key position new token tq sees
    u32x4_t qf[D / 16];                             // Q^T operand: d = 16 kk + 8 h .. +8
    {
        const uint16_t *qp = a.q + (((size_t)b * TQ + tq) * a.Hq + hq) * D + 8 * h;
        const uint32_t flip = neg ? 0x80008000u : 0u;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const u32x4_t x = *reinterpret_cast<const u32x4_t *>(qp + 16 * kk) ^ flip;
            qf[kk] = col_ok ? x : u32x4_t{0, 0, 0, 0};
        }
    }

    // ---- K/V stream ----------------------------------------------------
    // A step's loads are four block-loads: the K or the V rows (this KV head)
    // of the step's cache block bb, that is loads bb kDpb .. bb kDpb + kDpb - 1
    // of the K or V slot; load i fills LDS bytes [1024 i, 1024 i + 1024),
    // lane l row rows_per_dma i + l / cpr of the step at chunk position
    // l % cpr.  Wave w issues block-loads w, w + NC, ...: with four waves one
    // each (K0, K1, V0, V1), with two the K and V of block w.  Either way a
    // wave needs the id and descriptor span of one cache block, bb = w % 2.
    constexpr int kDpb = kBS / T::rows_per_dma;    // loads per block-load
    static_assert((NC == 2 || NC == 4) && 2 * T::dmas == 4 * kDpb, "block-loads split evenly over the waves, one block per wave");
    const int bb = wave & 1;
    const uint32_t row_stride = (uint32_t)(a.Hkv * T::row_bytes);
    const uint32_t blk_bytes = (uint32_t)kBS * row_stride;
    uint32_t voff[kDpb];
#pragma unroll
    for (int k = 0; k < kDpb; ++k) {
        const int R = T::rows_per_dma * k + lane / T::cpr;     // row of the block (the swizzle has period 16)
        voff[k] = (uint32_t)R * row_stride + (uint32_t)T::swz(R, lane % T::cpr) * 16u;
    }
    const int32_t __attribute__((address_space(4))) *tb =
        (const int32_t __attribute__((address_space(4))) *)(a.block_table + (size_t)b * a.max_blocks);
    // Physical id of block bb of step s (read through the scalar cache; an
    // index clamped into the table row, the value only used for rows that
    // exist).
    auto lookup = [&](int s) __attribute__((always_inline)) {
        return a.max_blocks > 0 ? tb[min(blk0 + 2 * s + bb, a.max_blocks - 1)] : 0;
    };
    // Byte offset and size of block bb of step s (physical id p) for this KV
    // head: rows past the chunk fall outside the size and read zero; an id
    // outside the pool marks the sequence bad and reads nothing.  Branch-free:
    // an unused block gets id 0 and size 0.  A sequence is bad for the whole
    // workgroup: the flags of the two blocks are combined after the stream.
    const size_t hk_off = (size_t)hk * T::row_bytes;
    auto span = [&](int s, int p, size_t &off, uint32_t &num) __attribute__((always_inline)) {
        int rows = t_end - kBS * (blk0 + 2 * s + bb);
        rows = rows < 0 ? 0 : (rows > kBS ? kBS : rows);
        rows = s < nsteps ? rows : 0;
        const bool wrong = (rows > 0) & ((uint32_t)p >= (uint32_t)a.num_blocks);
        bad = bad | wrong;
        const bool use = (rows > 0) & !wrong;
        off = (size_t)(use ? (uint32_t)p : 0u) * blk_bytes + hk_off;
        num = use ? (uint32_t)(rows - 1) * row_stride + T::row_bytes : 0u;
    };
    int id_next = lookup(0);
    // Queue this wave's block-loads of step s into (ks, vs); the id of step
    // s + 1 is read meanwhile.
    auto issue = [&](int s, uint8_t *ks, uint8_t *vs) __attribute__((always_inline)) {
        size_t off;
        uint32_t num;
        span(s, id_next, off, num);
#pragma unroll
        for (int j = 0; j < 4 / NC; ++j) {
            const bool is_v = ((wave + NC * j) >> 1) != 0;    // uniform
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(static_cast<const char *>(is_v ? a.v_cache : a.k_cache) + off, num);
            uint8_t *dst = (is_v ? vs : ks) + 1024 * kDpb * bb;
#pragma unroll
            for (int k = 0; k < kDpb; ++k) buffer_load_lds16(r, dst + 1024 * k, voff[k]);
        }
        id_next = lookup(s + 1);
    };

    // ---- LDS read offsets (bytes) ---------------------------------------
    // K operand of S^T = K Q^T: token row l32, d = 16 kk + 8 h .. +8 (bf16:
    // chunk 2 kk + h; e4m3: half h of chunk kk).
    int k_rd[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        k_rd[kk] = EB == 2 ? l32 * T::row_bytes + T::swz(l32, 2 * kk + h) * 16
                           : l32 * T::row_bytes + T::swz(l32, kk) * 16 + 8 * h;
    // V^T operand via transposing reads: within 16-lane group (hh, dh),
    // source lane s16 points at token row 4 hh + 8 t + s16 / 4 and
    // d = 32 db + 16 dh + 4 (s16 % 4); the second 16 tokens are 16 rows on.
    const int s16 = lane & 15, g16 = lane >> 4, hh = g16 >> 1, dh = g16 & 1;
    int v_rd[2][D / 32];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int r = 4 * hh + 8 * t + (s16 >> 2);
            const int d = 32 * db + 16 * dh + 4 * (s16 & 3);
            v_rd[t][db] = r * TB::row_bytes + TB::swz(r, d >> 3) * 16 + (d & 7) * 2;
        }

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m = kNegInf;       // exponent reference (log2 domain) of this column
    float lsum = 0.f;        // this lane's share of the column's sum

    // One step from (ks, vs): scores, softmax, PV.
    // e4m3: wave w widens rows [w 32 / NC, (w + 1) 32 / NC) of the V slot,
    // 16 values (one chunk) per lane and pass, into cv in the bf16 layout.
    auto widen_v = [&](const uint8_t *vs) __attribute__((always_inline)) {
        if constexpr (EB == 1) {
            constexpr int RPW = kStep / NC, PASSES = RPW * T::cpr / 64;
            static_assert(RPW * T::cpr % 64 == 0, "whole passes");
#pragma unroll
            for (int i = 0; i < PASSES; ++i) {
                const int q = lane + 64 * i;
                const int r = wave * RPW + q / T::cpr, c = q % T::cpr;
                const u32x4_t x = *reinterpret_cast<const u32x4_t *>(vs + r * T::row_bytes + T::swz(r, c) * 16);
                const u32x2_t a0 = fp8x4_to_bf16(x[0]), a1 = fp8x4_to_bf16(x[1]);
                const u32x2_t a2 = fp8x4_to_bf16(x[2]), a3 = fp8x4_to_bf16(x[3]);
                *reinterpret_cast<u32x4_t *>(cv + r * TB::row_bytes + TB::swz(r, 2 * c) * 16) =
                    u32x4_t{a0[0], a0[1], a1[0], a1[1]};
                *reinterpret_cast<u32x4_t *>(cv + r * TB::row_bytes + TB::swz(r, 2 * c + 1) * 16) =
                    u32x4_t{a2[0], a2[1], a3[0], a3[1]};
            }
        }
    };

    // The schedule is fenced: every K read before the first QK product
    // (one LDS latency a step instead of one per pair of products), and
    // every V^T read issued behind the QK products so that the softmax hides
    // its latency.
    auto compute = [&](int s, const uint8_t *ks, const uint8_t *vs) __attribute__((always_inline)) {
        f32x16_t sc;
        u32x4_t vf[2][D / 32];
        {
            u32x4_t kf[D / 16];
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                if constexpr (EB == 2) {
                    kf[kk] = *reinterpret_cast<const u32x4_t *>(ks + k_rd[kk]);
                } else {
                    const u32x2_t x = *reinterpret_cast<const u32x2_t *>(ks + k_rd[kk]);
                    const u32x2_t lo = fp8x4_to_bf16(x[0]), hi = fp8x4_to_bf16(x[1]);
                    kf[kk] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                sc = mfma_32x32x16_bf16(kf[kk], qf[kk], kk == 0 ? f32x16_t{} : sc);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int e = 16 * cc * TB::row_bytes;
                const uint8_t *vb = EB == 2 ? vs : cv;
                const u32x2_t lo = lds_read_tr16(reinterpret_cast<const uint16_t *>(vb + v_rd[0][db] + e));
                const u32x2_t hi = lds_read_tr16(reinterpret_cast<const uint16_t *>(vb + v_rd[1][db] + e));
                vf[cc][db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
            }
        __builtin_amdgcn_sched_barrier(0);
        // Lane (h, l32) holds tokens 8 (v / 4) + 4 h + v % 4 of the step.
        const int tok0 = kBS * (blk0 + 2 * s);
        if (tok0 + kStep > t_end || (TQ > 1 && tok0 + kStep - 1 > ctx - TQ)) {
            const int lim_l = min(t_end - 1, lim) - tok0 - 4 * h;   // last visible row, less 4 h
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 8 * (v >> 2) + (v & 3);
                sc[v] = r <= lim_l ? sc[v] : kNegInf;
            }
        }
        float mp[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
        for (int v = 0; v < 16; ++v) mp[v & 3] = fmaxf(mp[v & 3], sc[v]);
        float mraw = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
        mraw = pair_max_halves(mraw);
        const float mx = mraw == kNegInf ? kNegInf : mraw * c;
        const float m_new = fmaxf(m, mx);
        const bool grow = m_new > m + 8.0f;
        if (wave_any(grow)) {
            const float alpha = grow ? exp2_fast(m - m_new) : 1.0f;
            m = grow ? m_new : m;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        }
        const float nm = (m == kNegInf) ? 0.f : -m;
        u32x4_t pk[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = exp2_fast(__builtin_fmaf(sc[8 * cc + 2 * e], c, nm));
                const float p1 = exp2_fast(__builtin_fmaf(sc[8 * cc + 2 * e + 1], c, nm));
                pk[cc][e] = pack_bf16x2(p0, p1);
                lsum += p0 + p1;
            }
        // O^T += V^T P^T over the step's two 16-token halves; the S^T
        // accumulator is the B operand once each product takes its tokens in
        // the accumulator's order.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] = mfma_32x32x16_bf16(vf[cc][db], pk[cc], oacc[db]);
    };

    // Step s: wait for its loads (this wave's, then everyone's via the
    // barrier, which also frees the slot read at step s - 1), queue step
    // s + NS - 1 into that freed slot, compute step s.  Every step queues
    // exactly one step's loads (past the chunk they fetch nothing and fill
    // zeros), so the count of loads left in flight at each wait is fixed.
    auto body = [&](int s, const uint8_t *ks, const uint8_t *vs, uint8_t *kn, uint8_t *vn) __attribute__((always_inline)) {
        wait_vmcnt<(NS - 2) * LPW, true>();
        plain_barrier();
        issue(s + NS - 1, kn, vn);
        if constexpr (EB == 1) {
            // Widen this wave's share of the step's V rows into cv (free:
            // every wave passed the barrier after its last reads of it),
            // then wait for the other waves' shares.
            widen_v(vs);
            wait_lgkm0();
            plain_barrier();
        }
        compute(s, ks, vs);
    };
    issue(0, k0, v0);
    if constexpr (NS == 3) {
        __shared__ __attribute__((aligned(1024))) uint8_t k2[T::slot_bytes];
        __shared__ __attribute__((aligned(1024))) uint8_t v2[T::slot_bytes];
        issue(1, k1, v1);
        for (int s = 0; s < nsteps; s += 3) {
            body(s, k0, v0, k2, v2);
            if (s + 1 < nsteps) body(s + 1, k1, v1, k0, v0);
            if (s + 2 < nsteps) body(s + 2, k2, v2, k1, v1);
        }
    } else {
        for (int s = 0; s < nsteps; s += 2) {
            body(s, k0, v0, k1, v1);
            if (s + 1 < nsteps) body(s + 1, k1, v1, k0, v0);
        }
    }
    // The trailing loads (past the chunk: zero fills) land and every wave is
    // done with the ring before the next item's first loads go there.  The
    // same barrier combines the waves' bad-id flags (each wave checked one of
    // the two blocks of every step): written before it, read after it, and
    // written again only after the next item's first barrier, which every
    // wave reaches after its read.
    if (lane == 0) bad_s[wave] = bad ? 1 : 0;
    wait_vmcnt<0, true>();
    plain_barrier();
#pragma unroll
    for (int w = 0; w < NC; ++w) bad = bad | (bad_s[w] != 0);
    if (DYN && threadIdx.x == 0) ticket = atomicAdd(a.work_ctr, 1u);

    // ---- output ------------------------------------------------------------
    const float ltot = pair_sum_halves(lsum);
    if (col_ok) {
    const float lse = bad ? __builtin_nanf("") : (ltot > 0.f ? (m + __log2f(ltot)) * kLn2 : kNegInf);
    const float inv = bad ? __builtin_nanf("") : (ltot > 0.f ? a.v_scale / ltot : 0.f);
    const size_t orow = ((size_t)b * TQ + tq) * a.Hq + hq;
    // Lane (h, l32) holds d = 32 db + 8 g4 + 4 h .. +3 of its column.
    if (a.splits == 1) {
        uint16_t *dst = a.o + orow * D + 4 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const u32x2_t w = {pack_bf16x2(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv),
                                   pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
                *reinterpret_cast<u32x2_t *>(dst + 32 * db + 8 * g4) = w;
            }
        if (h == 0 && a.lse != nullptr) a.lse[((size_t)b * a.Hq + hq) * TQ + tq] = lse;
    } else {
        const size_t row = orow * a.splits + split;
        float *dst = a.part_o + row * D + 4 * h;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *reinterpret_cast<f32x4_t *>(dst + 32 * db + 8 * g4) =
                    f32x4_t{oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv, oacc[db][4 * g4 + 2] * inv,
                            oacc[db][4 * g4 + 3] * inv};
        if (h == 0) a.part_lse[row] = lse;
    }
    }   // col_ok
    }   // items
}

// Two ring slots: a third (loads two steps ahead) measured no faster.
constexpr int kRing = 2;

// Dynamic LDS (unused by the kernel) that limits how many workgroups share a
// CU.  Measured on MI355X: 64-column workgroups at D = 128 run 1.5-3.5%
// faster two to a CU (54 KiB each) than four (batch 64 with 16 new tokens,
// 128K context with 8); 128-column workgroups are 35-45% slower alone on a
// CU than two to a CU (their register use allows two), and keep that.
template <int D, int NC, int EB>
constexpr unsigned wide_pad() { return (D == 128 && NC == 2 && EB == 2) ? 22528u : 0u; }

// Workgroups of one instance resident on a CU at once (queried once).
template <int D, int NC, bool DYN, int EB>
int wide_resident_per_cu()
{
    static const int n = [] {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, reinterpret_cast<const void *>(&decode_wide_kernel<D, NC, kRing, DYN, EB>),
                                                         64 * NC, wide_pad<D, NC, EB>()) != hipSuccess || v <= 0)
            v = 1;
        return v;
    }();
    return n;
}

template <int D, int NC, int EB>
hipError_t launch_nc(const DecodeArgs &a, hipStream_t s)
{
    const long long units = (long long)a.B * a.Hkv * a.splits;
    const long long GT = (long long)(a.Hq / a.Hkv) * a.T;
    const long long n_grp = (GT + kColsPerWave * NC - 1) / (kColsPerWave * NC);
    if (units <= 0 || n_grp <= 0) return hipSuccess;
    constexpr unsigned pad = wide_pad<D, NC, EB>();
    if (n_grp == 1) {
        // As many workgroups as the GPU holds at once (never more than the
        // items), each taking items until the counter passes the last one.
        const long long grid = std::min<long long>(units, (long long)wide_resident_per_cu<D, NC, true, EB>() * compute_units());
        hipLaunchKernelGGL((decode_wide_kernel<D, NC, kRing, true, EB>), dim3((unsigned)grid), dim3(64 * NC), pad, s, a);
    } else {
        const long long grid = (units + 7) / 8 * 8 * n_grp;   // ids padded to whole rounds over the XCDs
        hipLaunchKernelGGL((decode_wide_kernel<D, NC, kRing, false, EB>), dim3((unsigned)grid), dim3(64 * NC), pad, s, a);
    }
    return hipGetLastError();
}

}  // namespace

// bf16 caches from 33 columns on; e4m3 caches (head_dim 128) from 65: at 64
// columns the 16-column tiles measured faster there (128K context, 8 new
// tokens: 0.322 against 0.338 ms), at 128 and 256 the wide kernel (0.617 ->
// 0.396 ms and 1.115 -> 0.728 ms).
bool decode_wide_supported(int head_dim, bool kv_fp8, long long columns)
{
    if (kv_fp8) return head_dim == 128 && columns > 64;
    return (head_dim == 128 || head_dim == 64) && columns > 32;
}

hipError_t launch_decode_wide(const DecodeArgs &a, int head_dim, bool kv_fp8, hipStream_t s)
{
    const long long GT = (long long)(a.Hq / a.Hkv) * a.T;
    if (kv_fp8) return head_dim == 128 && GT > 64 ? launch_nc<128, 4, 1>(a, s) : hipErrorInvalidValue;
    if (head_dim == 128) return GT <= 64 ? launch_nc<128, 2, 2>(a, s) : launch_nc<128, 4, 2>(a, s);
    if (head_dim == 64) return GT <= 64 ? launch_nc<64, 2, 2>(a, s) : launch_nc<64, 4, 2>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
