// prefill_bf16.hip -- exact attention forward, bf16 in/out, fp32 softmax and
// accumulation, on the gfx950 matrix cores.
//
// The FlashAttention scheme as the pages describe it ("推理加速" interview
// notes, section FlashAttention: cut Q/K/V into blocks, load blocks on chip,
// compute block attention there, online softmax, write back only the final
// output; chenyy20.com "抱infra脚", Flash Attention 基本原理 / 核心技术:
// tiling, online softmax, fusion of QK + softmax + PV; "GPU Kernel 调度：
// 大模型推理的拐点 2026", FlashAttention evolution: query blocks in parallel,
// K/V blocks pipelined, row-max / row-sum reductions):
//
//   one workgroup = 128 query rows of one (batch, query head), 4 waves of 32
//   rows each.  K/V tiles of 64 keys stream through a two-stage LDS ring fed
//   by buffer loads that write LDS directly (no register staging; rows past
//   the end of the sequence read as zero), so tile j+1 is in flight while
//   tile j is computed.  Per tile and wave:
//     S^T = K Q^T          32x32x16 bf16 MFMA; one lane = one query row, so
//                          the row max is an in-lane reduction plus one
//                          exchange between the two wave halves
//     causal / ragged mask only on tiles that cross the diagonal or the end
//     online softmax       exp2 domain: p = 2^(s * scale*log2e - m) is one
//                          FMA + one v_exp_f32 per score.  Lazy rescaling:
//                          the exponent reference m only moves when the row
//                          max has grown by more than 2^8, so most tiles skip
//                          rescaling O; the result is the same up to rounding
//     P -> bf16 (RNE)      kept in registers; the S^T accumulator layout is
//                          the B operand of O^T = V^T P^T once the keys of
//                          each MFMA are taken in the accumulator's order.
//                          The row sum l accumulates the fp32 P, so lse keeps
//                          fp32 accuracy
//     O^T += V^T P^T       32x32x16 bf16 MFMA; V stays row-major in LDS and
//                          its transposed operand comes from ds_read_b64_tr_b16
//   Epilogue: O = O / l rounded to bf16, lse = (m + log2 l) * ln 2.
//
// LDS tiles are row-major with 16-byte chunks XOR-swizzled per row so that
// both the K row reads and the transposing V reads spread over all banks.
//
// Grid: one workgroup per (q-tile, query head, batch).  Workgroup ids are
// mapped so that the longest causal q-tiles start first and all query heads
// of one (batch, KV head) land on the same XCD (ids go round-robin over the
// 8 XCDs), where its K/V stays in that XCD's L2.
#include <type_traits>

#include "gfx950.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBR = 128;      // query rows per workgroup
constexpr int kBC = 64;       // keys per K/V tile
constexpr int kBS = 16;       // tokens per cache block (paged keys and values)
constexpr int kThreads = 256;
constexpr int kWaves = 4;

// An empty volatile asm statement: placed inside a rarely taken branch it
// keeps the compiler from turning the branch into unconditional arithmetic.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

template <int D>
struct Tile {
    static constexpr int cpr = D / 8;                     // 16-byte chunks per row
    static constexpr int elems = kBC * D;                 // bf16 elements per K or V tile
    static constexpr int loads_per_wave = kBC * cpr / 64 / kWaves;   // 1 KiB LDS-direct loads
    // Physical chunk of logical chunk c in row r.
    static __device__ __forceinline__ int swz(int r, int c)
    {
        if constexpr (D == 128)
            return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
        else
            return c ^ ((r >> 1) & 7);
    }
};

__device__ __forceinline__ void map_workgroup(int L, const PrefillArgs &a, int n_qtiles,
                                              int &b, int &hq, int &qt)
{
    const int G = a.Hq / a.Hkv;
    const int groups = a.B * a.Hkv;                 // (batch, KV head) pairs
    int qt_rev, g, hg;
    if (groups % 8 == 0) {
        const int xcd = L & 7, r = L >> 3;
        const int per = (groups >> 3) * G;          // workgroups per XCD per q-tile
        qt_rev = r / per;
        const int rem = r - qt_rev * per;
        g = xcd + 8 * (rem / G);
        hg = rem % G;
    } else {
        const int per = groups * G;
        qt_rev = L / per;
        const int rem = L - qt_rev * per;
        g = rem / G;
        hg = rem % G;
    }
    b = g / a.Hkv;
    hq = (g % a.Hkv) * G + hg;
    qt = n_qtiles - 1 - qt_rev;
}

template <int D, bool CAUSAL, bool PAGED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_kernel(PrefillArgs a, int n_qtiles)
{
    using T = Tile<D>;
    __shared__ __attribute__((aligned(1024))) uint16_t k_st0[T::elems];
    __shared__ __attribute__((aligned(1024))) uint16_t v_st0[T::elems];
    __shared__ __attribute__((aligned(1024))) uint16_t k_st1[T::elems];
    __shared__ __attribute__((aligned(1024))) uint16_t v_st1[T::elems];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;

    int b, hq, qt;
    map_workgroup(blockIdx.x, a, n_qtiles, b, hq, qt);
    const int G = a.Hq / a.Hkv, hk = hq / G;
    const int i0 = qt * kBR;
    const int q0 = i0 + wave * 32;      // first query row of this wave (uniform)
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

    int kend = Sk;                      // keys [0, kend) may be visible to this workgroup
    if (CAUSAL) kend = min(Sk, min(a.Sq, i0 + kBR) + diag);
    const int ntiles = kend > 0 ? (kend + kBC - 1) / kBC : 0;

    // Exponent scale c = scale * log2(e), made non-negative by flipping the
    // sign of Q (exact in bf16) when the caller's scale is negative.
    const bool neg = a.scale_log2 < 0.f;
    const float c = neg ? -a.scale_log2 : a.scale_log2;

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
    const size_t head_off = PAGED ? 0 : ((size_t)b * a.Sk * a.Hkv + hk) * D;      // elements
    const char *kbase = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.k) + head_off);
    const char *vbase = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.v) + head_off);
    // Bytes from this head's first key to the end of its last key row.
    const uint32_t span = Sk > 0 ? (uint32_t)(((size_t)(Sk - 1) * a.Hkv * D + D) * 2) : 0u;

    // Per-lane source offsets (bytes, relative to the tile's first key) of the
    // 16-byte chunks this lane's LDS-direct loads deliver: load i of wave w
    // fills LDS chunk slots (w * loads + i) * 64 + lane.
    uint32_t src_off[T::loads_per_wave];
#pragma unroll
    for (int i = 0; i < T::loads_per_wave; ++i) {
        const int slot = (wave * T::loads_per_wave + i) * 64 + lane;
        const int r = slot / T::cpr, p = slot % T::cpr;
        const int cl = T::swz(r, p);                      // swz is an involution
        // Paged: the wave's 16 rows are one cache block; offsets are relative
        // to this head's slice of that block's first token.
        src_off[i] = (uint32_t)(PAGED ? r - kBS * wave : r) * row_bytes + (uint32_t)cl * 16u;
    }

    // Paged: wave w loads cache block 4 j + w of tile j (its 16 rows).  The
    // physical block ids come through the scalar cache one tile ahead.
    const int n_lblocks = (Sk + kBS - 1) / kBS;
    const int32_t __attribute__((address_space(4))) *tb =
        (const int32_t __attribute__((address_space(4))) *)(a.block_table + (PAGED ? (size_t)b * a.max_blocks : 0));
    int phys_next = (PAGED && wave < n_lblocks) ? tb[wave] : 0;
    const uint32_t blk_bytes = (uint32_t)kBS * row_bytes;

    auto issue_tile = [&](int j, uint16_t *ks, uint16_t *vs) __attribute__((always_inline)) {
        __amdgpu_buffer_rsrc_t rk, rv;
        if constexpr (PAGED) {
            const int lb = (kBC / kBS) * j + wave;
            const int p = phys_next;
            phys_next = lb + kBC / kBS < n_lblocks ? tb[lb + kBC / kBS] : 0;
            int valid = min(kBS, Sk - kBS * lb);
            long long phys = 0;
            if (valid > 0) {
                if (p < 0 || p >= a.num_blocks) {
                    bad = true;
                    valid = 0;
                } else {
                    phys = p;
                }
            } else {
                valid = 0;
            }
            const size_t off = (size_t)phys * blk_bytes + (size_t)hk * D * 2;
            const uint32_t num = valid > 0 ? (uint32_t)(valid - 1) * row_bytes + D * 2 : 0u;
            rk = make_rsrc(static_cast<const char *>(a.k) + off, num);
            rv = make_rsrc(static_cast<const char *>(a.v) + off, num);
        } else {
            const uint32_t start = (uint32_t)(j * kBC) * row_bytes;
            const uint32_t left = span > start ? span - start : 0u;
            rk = make_rsrc(kbase + start, left);
            rv = make_rsrc(vbase + start, left);
        }
#pragma unroll
        for (int i = 0; i < T::loads_per_wave; ++i) {
            const int chunk0 = (wave * T::loads_per_wave + i) * 64;      // uniform
            buffer_load_lds16(rk, ks + chunk0 * 8, src_off[i]);
            buffer_load_lds16(rv, vs + chunk0 * 8, src_off[i]);
        }
    };

    // ---- per-lane LDS read offsets (elements) --------------------------------
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

    // ---- per-lane softmax state and output accumulator ----------------
    f32x16_t oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m = kNegInf;      // exponent reference (log2 domain) of this row
    float lsum = 0.f;       // this lane's share of the row sum
    const f32x16_t zero16 = {};

    // Tiles before `first_masked` are fully visible to every row of this wave.
    int first_masked = Sk / kBC;                         // full tiles inside the sequence
    if (CAUSAL) first_masked = min(first_masked, max(0, (q0 + diag + 1) / kBC));

    // One code path for every tile: masking is a uniform branch around the
    // few instructions that need it, so the output accumulator keeps its
    // registers across tiles.
    auto run_tile = [&](const uint16_t *ks, const uint16_t *vs, int j, auto masked_tag) __attribute__((always_inline)) {
        constexpr bool masked = decltype(masked_tag)::value;
        const int kv0 = j * kBC;
        // S^T = K Q^T (both 32-key halves; on diagonal tiles a half may be
        // fully masked, which the mask below handles)
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = mfma_32x32x16_bf16(*reinterpret_cast<const u32x4_t *>(ks + k_rd[0] + 32 * kb * D), qf[0], zero16);
#pragma unroll
            for (int kk = 1; kk < D / 16; ++kk) {
                const u32x4_t kop = *reinterpret_cast<const u32x4_t *>(ks + k_rd[kk] + 32 * kb * D);
                s[kb] = mfma_32x32x16_bf16(kop, qf[kk], s[kb]);
            }
        }
        if constexpr (masked) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = kv0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
                    const bool vis = key < Sk && (!CAUSAL || key <= my_q + diag);
                    s[kb][v] = vis ? s[kb][v] : kNegInf;
                }
        }
        // Row max of the raw scores (c >= 0, so scaling preserves order).
        float mraw = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) mraw = fmaxf(mraw, s[kb][v]);
        mraw = pair_max_halves(mraw);
        const float mx = mraw == kNegInf ? kNegInf : mraw * c;
        const float m_new = fmaxf(m, mx);
        const bool grow = m_new > m + 8.0f;
        if (wave_any(grow)) {
            keep_branch();
            const float alpha = grow ? exp2_fast(m - m_new) : 1.0f;
            m = grow ? m_new : m;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        }
        const float nm = (m == kNegInf) ? 0.f : -m;
        // Exponents s c - m; masked scores stay -inf (also when c == 0).
        float x[2][16];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) x[kb][v] = __builtin_fmaf(s[kb][v], c, nm);
        if constexpr (masked) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) x[kb][v] = s[kb][v] == kNegInf ? kNegInf : x[kb][v];
        }
        // P = 2^x -> bf16 pairs; the row sum adds the fp32 values.
        u32x4_t pk[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = exp2_fast(x[kb][8 * cc + 2 * e]), p1 = exp2_fast(x[kb][8 * cc + 2 * e + 1]);
                    pk[kb][cc][e] = pack_bf16x2(p0, p1);
                    lsum += p0 + p1;
                }
        // O^T += V^T P^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int kbase_el = (32 * kb + 16 * cc) * D;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const u32x2_t lo = lds_read_tr16(vs + v_rd[0][db] + kbase_el);
                    const u32x2_t hi = lds_read_tr16(vs + v_rd[1][db] + kbase_el);
                    const u32x4_t vop = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[db] = mfma_32x32x16_bf16(vop, pk[kb][cc], oacc[db]);
                }
            }
        }
    };

    // Tiles [0, fm) need no mask for this wave: they run in a branch-free
    // loop over the two static stages.  The remaining tiles (those crossing
    // the diagonal or the end of the keys, and an odd leftover) run through
    // the masked body.  Every wave passes one barrier per tile either way.
    const int fm = min(first_masked, ntiles);
    if (ntiles > 0) issue_tile(0, k_st0, v_st0);
    __syncthreads();
    int j = 0;
    for (; j + 1 < fm; j += 2) {
        issue_tile(j + 1, k_st1, v_st1);
        run_tile(k_st0, v_st0, j, std::false_type{});
        __syncthreads();
        if (j + 2 < ntiles) issue_tile(j + 2, k_st0, v_st0);
        run_tile(k_st1, v_st1, j + 1, std::false_type{});
        __syncthreads();
    }
    for (; j < ntiles; ++j) {
        uint16_t *ks = (j & 1) ? k_st1 : k_st0, *vs = (j & 1) ? v_st1 : v_st0;
        if (j + 1 < ntiles) issue_tile(j + 1, (j & 1) ? k_st0 : k_st1, (j & 1) ? v_st0 : v_st1);
        run_tile(ks, vs, j, std::true_type{});
        __syncthreads();
    }

    // ---- epilogue ----------------------------------------------------------
    if constexpr (PAGED) bad = __syncthreads_or(bad);
    const float ltot = pair_sum_halves(lsum);
    if (my_q < a.Sq) {
        float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
        if (PAGED && bad) inv = __builtin_nanf("");
        uint16_t *op = static_cast<uint16_t *>(a.o) + (((size_t)b * a.Sq + my_q) * a.Hq + hq) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * db + 8 * g4 + 4 * h;
                const u32x2_t w = {pack_bf16x2(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv),
                                   pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
                *reinterpret_cast<u32x2_t *>(op + d0) = w;
            }
        }
        if (a.lse != nullptr && h == 0)
            a.lse[((size_t)b * a.Hq + hq) * a.Sq + my_q] =
                (PAGED && bad) ? __builtin_nanf("") : (ltot > 0.f ? (m + __log2f(ltot)) * kLn2 : kNegInf);
    }
}

template <int D, bool CAUSAL, bool PAGED>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s)
{
    const int n_qtiles = (a.Sq + kBR - 1) / kBR;
    const long long grid = (long long)n_qtiles * a.Hq * a.B;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, PAGED>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, n_qtiles);
    return hipGetLastError();
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
