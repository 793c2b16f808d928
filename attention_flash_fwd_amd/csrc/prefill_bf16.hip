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
//   rows each.  K/V tiles of 64 keys stream through a two-stage LDS ring;
//   while the matrix cores work on tile j the next tile's global loads are in
//   flight.  Per tile and wave:
//     S^T = K Q^T         (32x32x16 bf16 MFMA; one lane = one query row, so
//                          the row max / row sum are in-lane reductions plus
//                          one exchange between the two wave halves)
//     causal / ragged mask (only on tiles that cross the diagonal or the end)
//     online softmax in the exp2 domain (scale*log2e folded into one multiply)
//                          with lazy rescaling: the running max used as the
//                          exponent reference only moves when the true max
//                          has grown by more than 2^8, so most tiles skip the
//                          O rescale; results are identical up to rounding
//     P -> bf16 (RNE), kept in registers: the S^T accumulator layout is
//                          exactly the B-operand layout of O^T = V^T P^T once
//                          the keys are permuted consistently in V^T
//     O^T += V^T P^T      (32x32x16 bf16 MFMA, V stored transposed in LDS)
//   Epilogue: O = O / l rounded to bf16, lse = (m + log2 l) * ln 2.
//
// Grid: one workgroup per (q-tile, query head, batch).  Workgroup ids are
// mapped so that the longest causal q-tiles start first and all query heads
// of one (batch, KV head) land on the same XCD (ids go round-robin over the
// 8 XCDs), where its K/V stays in that XCD's L2.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBR = 128;      // query rows per workgroup
constexpr int kBC = 64;       // keys per K/V tile
constexpr int kThreads = 256;

template <int D>
struct Smem {
    static constexpr int kPitch = D + 8;            // K row pitch (bf16), breaks bank aliasing
    static constexpr int vPitch = kBC + 8;          // V^T row pitch (bf16)
    static constexpr int kElems = kBC * kPitch;
    static constexpr int vElems = D * vPitch;
    static constexpr int stage = kElems + vElems;   // one K tile + one V^T tile
    static constexpr int kChunks = kBC * D / 8 / kThreads;  // 16-byte K chunks per thread
};

// Position of key kappa (0..63 in a tile) inside a V^T row: bits 2 and 3 of
// the key index trade places.  The score accumulator of lane half h holds,
// for each 16-key MFMA chunk, keys {8j + 4h + r}; with this permutation those
// eight keys sit contiguously at 8h + 4j + r, so one 16-byte LDS read gives
// the matching V^T operand.
__device__ __forceinline__ int vt_pos(int kappa)
{
    return (kappa & ~0xC) | ((kappa & 4) << 1) | ((kappa & 8) >> 1);
}

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

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_kernel(PrefillArgs a, int n_qtiles)
{
    using SM = Smem<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SM::stage];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;

    int b, hq, qt;
    map_workgroup(blockIdx.x, a, n_qtiles, b, hq, qt);
    const int G = a.Hq / a.Hkv, hk = hq / G;
    const int i0 = qt * kBR;
    const int q0 = i0 + wave * 32;      // first query row of this wave
    const int my_q = q0 + l32;          // query row of this lane
    const int diag = a.Sk - a.Sq;       // key j visible to row i iff j <= i + diag

    int kend = a.Sk;                    // keys [0, kend) may be visible to this workgroup
    if (CAUSAL) kend = min(a.Sk, min(a.Sq, i0 + kBR) + diag);
    const int ntiles = kend > 0 ? (kend + kBC - 1) / kBC : 0;

    const uint16_t *__restrict__ qg = static_cast<const uint16_t *>(a.q);
    const uint16_t *__restrict__ kg = static_cast<const uint16_t *>(a.k);
    const uint16_t *__restrict__ vg = static_cast<const uint16_t *>(a.v);

    // Q^T operand of S^T = K Q^T: lane (h, l32) holds q[my_q][16ks + 8h .. +8].
    u32x4_t qf[D / 16];
    {
        const size_t row = ((size_t)b * a.Sq + my_q) * a.Hq + hq;
        const uint16_t *qp = qg + row * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qf[ks] = my_q < a.Sq ? *reinterpret_cast<const u32x4_t *>(qp + 16 * ks) : u32x4_t{0, 0, 0, 0};
    }

    const size_t kv_rs = (size_t)a.Hkv * D;         // elements between consecutive keys
    const uint16_t *kbase = kg + (size_t)b * a.Sk * kv_rs + (size_t)hk * D;
    const uint16_t *vbase = vg + (size_t)b * a.Sk * kv_rs + (size_t)hk * D;

    // ---- K/V tile staging: global -> registers -> LDS ------------------
    u32x4_t kreg[SM::kChunks];
    u32x4_t vreg[4];
    const bool v_loader = tid < 16 * (D / 8);       // (key quad, 8-wide d chunk) items
    const int v_kq = tid & 15, v_dc = tid >> 4;

    auto load_tile = [&](int j) {
        const int kv0 = j * kBC;
#pragma unroll
        for (int i = 0; i < SM::kChunks; ++i) {
            const int c = tid + kThreads * i;
            const int row = c / (D / 8), col = c % (D / 8);
            const int key = kv0 + row;
            kreg[i] = key < a.Sk ? *reinterpret_cast<const u32x4_t *>(kbase + key * kv_rs + col * 8)
                                 : u32x4_t{0, 0, 0, 0};
        }
        if (v_loader) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kv0 + 4 * v_kq + r;
                vreg[r] = key < a.Sk ? *reinterpret_cast<const u32x4_t *>(vbase + key * kv_rs + v_dc * 8)
                                     : u32x4_t{0, 0, 0, 0};
            }
        }
    };

    auto store_tile = [&](int stage) {
        uint16_t *ks = smem + stage * SM::stage;
        uint16_t *vs = ks + SM::kElems;
#pragma unroll
        for (int i = 0; i < SM::kChunks; ++i) {
            const int c = tid + kThreads * i;
            const int row = c / (D / 8), col = c % (D / 8);
            *reinterpret_cast<u32x4_t *>(ks + row * SM::kPitch + col * 8) = kreg[i];
        }
        if (v_loader) {
            // vreg[r] holds V[4kq + r][8dc .. 8dc+7]; write V^T rows 8dc .. 8dc+7,
            // four consecutive keys (8 bytes) per row.
            const int pos = vt_pos(4 * v_kq);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2_t lo = {pack_lo16(vreg[0][i], vreg[1][i]), pack_lo16(vreg[2][i], vreg[3][i])};
                const u32x2_t hi = {pack_hi16(vreg[0][i], vreg[1][i]), pack_hi16(vreg[2][i], vreg[3][i])};
                *reinterpret_cast<u32x2_t *>(vs + (8 * v_dc + 2 * i) * SM::vPitch + pos) = lo;
                *reinterpret_cast<u32x2_t *>(vs + (8 * v_dc + 2 * i + 1) * SM::vPitch + pos) = hi;
            }
        }
    };

    // ---- per-lane softmax state and output accumulator ----------------
    f32x16_t oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m = kNegInf;      // exponent reference (log2 domain) of this row
    float lsum = 0.f;       // this lane's share of the row sum

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        if (j + 1 < ntiles) load_tile(j + 1);

        const uint16_t *ks = smem + (j & 1) * SM::stage;
        const uint16_t *vs = ks + SM::kElems;
        const int kv0 = j * kBC;

        // Which 32-key halves of the tile can this wave see at all?
        bool blk_live[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int kstart = kv0 + 32 * kb;
            blk_live[kb] = kstart < a.Sk && (!CAUSAL || kstart <= q0 + 31 + diag);
        }

        // S^T = K Q^T for the live halves.
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
            if (blk_live[kb]) {
                const uint16_t *kr = ks + (32 * kb + l32) * SM::kPitch + 8 * h;
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk)
                    s[kb] = mfma_32x32x16_bf16(*reinterpret_cast<const u32x4_t *>(kr + 16 * kk), qf[kk], s[kb]);
            }
        }

        // Scale into the exp2 domain and mask where some key may be invisible.
        const bool need_mask = (kv0 + kBC > a.Sk) || (CAUSAL && kv0 + kBC - 1 > q0 + diag);
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float t = s[kb][v] * a.scale_log2;
                if (need_mask) {
                    const int key = kv0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
                    const bool vis = key < a.Sk && (!CAUSAL || key <= my_q + diag);
                    t = vis ? t : kNegInf;
                }
                s[kb][v] = t;
                mx = fmaxf(mx, t);
            }
        }
        mx = pair_max_halves(mx);

        // Online softmax with lazy rescaling of the exponent reference.
        const float m_new = fmaxf(m, mx);
        const bool grow = m_new > m + 8.0f;
        if (wave_any(grow)) {
            const float alpha = grow ? exp2_fast(m - m_new) : 1.0f;
            m = grow ? m_new : m;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
        }
        const float mref = (m == kNegInf) ? 0.f : m;

        // P = 2^(t - m), row-sum share, pack to bf16 as the PV B operand.
        u32x4_t pk[2][2];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = exp2_fast(s[kb][8 * c + 2 * e] - mref);
                    const float p1 = exp2_fast(s[kb][8 * c + 2 * e + 1] - mref);
                    rs += p0 + p1;
                    pk[kb][c][e] = pack_bf16x2(p0, p1);
                }
            }
        }
        lsum += rs;

        // O^T += V^T P^T over the live halves.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!blk_live[kb]) continue;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint16_t *vr = vs + l32 * SM::vPitch + 32 * kb + 16 * c + 8 * h;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    oacc[db] = mfma_32x32x16_bf16(*reinterpret_cast<const u32x4_t *>(vr + 32 * db * SM::vPitch),
                                                  pk[kb][c], oacc[db]);
            }
        }

        if (j + 1 < ntiles) store_tile((j + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue ----------------------------------------------------------
    const float ltot = pair_sum_halves(lsum);
    if (my_q < a.Sq) {
        const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
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
            a.lse[((size_t)b * a.Hq + hq) * a.Sq + my_q] = ltot > 0.f ? (m + __log2f(ltot)) * kLn2 : kNegInf;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s)
{
    const int n_qtiles = (a.Sq + kBR - 1) / kBR;
    const long long grid = (long long)n_qtiles * a.Hq * a.B;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, n_qtiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, bool causal, hipStream_t s)
{
    if (head_dim == 128) return causal ? launch_one<128, true>(a, s) : launch_one<128, false>(a, s);
    if (head_dim == 64) return causal ? launch_one<64, true>(a, s) : launch_one<64, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
