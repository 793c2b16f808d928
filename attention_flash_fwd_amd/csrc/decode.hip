// decode.hip -- single-token attention over a paged KV cache, Flash-Decoding
// style ("GPU Kernel 调度：大模型推理的拐点 2026", paragraphs on Flash Decoding
// and its cost: the cached K/V of a sequence is cut into chunks processed in
// parallel, each chunk yields a partial output with its log-sum-exp, and a
// small reduce kernel merges the partials with the online-softmax formula in
// fp32; chenyy20.com "抱infra脚", section Paged Attention: fixed-size blocks
// reached through a block table).
//
// Kernel 1, decode_split: one workgroup per (chunk, KV head, sequence).  The
//   G = Hq / Hkv query heads that share the KV head are packed as the columns
//   of 16x16x32 bf16 MFMAs, so each K/V byte is read from HBM once for all of
//   them.  The four waves of the workgroup take turns over pairs of 16-token
//   cache blocks; each wave keeps its own running max / sum and its partial
//   output, with the next pair's K/V loads in flight while the current pair
//   is computed.  K goes straight from global memory into MFMA A operands;
//   V is transposed through a wave-private LDS slab.  Tokens past the chunk
//   end are never read (their operands are zero), so unused cache slots may
//   hold anything.  The four wave partials are merged in LDS and the chunk's
//   normalised output and log-sum-exp are written as fp32.
// Kernel 2, decode_combine: one wave per (sequence, query head) merges the
//   chunk partials: M = max lse_s, w_s = e^(lse_s - M), O = sum w_s O_s / sum w_s,
//   lse = M + ln sum w_s; O rounded to bf16.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBS = 16;         // tokens per cache block
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int D>
struct DecodeSmem {
    static constexpr int pitch = D + 8;                 // V row pitch (bf16)
    static constexpr int slab = 2 * kBS * pitch;        // two blocks, per wave (bf16 elements)
    static constexpr int vbytes = kWaves * slab * 2;
    static constexpr int cbytes = kWaves * (16 * D + 32) * 4;   // partial O + m + l per wave
    static constexpr int bytes = vbytes > cbytes ? vbytes : cbytes;
};

template <int D>
__global__ void __launch_bounds__(kThreads) decode_split_kernel(DecodeArgs a)
{
    using SM = DecodeSmem<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[SM::bytes];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;

    const int split = blockIdx.x % a.splits;
    const int hk = (blockIdx.x / a.splits) % a.Hkv;
    const int b = blockIdx.x / (a.splits * a.Hkv);
    const int G = a.Hq / a.Hkv;

    const int ctx = a.ctx_lens[b];
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
    const int nsteps = (nblk + 1) / 2;                  // pairs of blocks

    // Q^T operand: lane (g, l16) holds q[head l16][32 kk + 8 g .. +8]; heads past G are 0.
    u32x4_t qf[D / 32];
    {
        const bool hv = l16 < G;
        const uint16_t *qp = a.q + ((size_t)b * a.Hq + hk * G + (hv ? l16 : 0)) * D + 8 * g;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
            qf[kk] = hv ? *reinterpret_cast<const u32x4_t *>(qp + 32 * kk) : u32x4_t{0, 0, 0, 0};
    }

    const size_t tok_rs = (size_t)a.Hkv * D;            // elements between tokens of a block
    const size_t blk_rs = (size_t)kBS * tok_rs;         // elements between blocks
    const int32_t *table = a.block_table + (size_t)b * a.max_blocks;

    // Loads of one step: blocks (blk0 + 2 st, +1); lane (g, l16) fetches token l16's
    // d-range 32 kk + 8 g .. +8 of K and V for each block.
    u32x4_t kc[2][D / 32], vc[2][D / 32];
    auto load_step = [&](int st, u32x4_t (&kr)[2][D / 32], u32x4_t (&vr)[2][D / 32], bool &oob) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int lb = 2 * st + p;                  // block index within the chunk
            int phys = -1;
            if (lb < nblk) phys = table[blk0 + lb];
            const bool in_pool = phys >= 0 && phys < a.num_blocks;
            if (lb < nblk && !in_pool) oob = true;
            const int tok = (blk0 + lb) * kBS + l16;
            const bool live = lb < nblk && in_pool && tok < t_end;
            const size_t base = (size_t)(in_pool ? phys : 0) * blk_rs + (size_t)l16 * tok_rs + (size_t)hk * D + 8 * g;
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                kr[p][kk] = live ? *reinterpret_cast<const u32x4_t *>(a.k_cache + base + 32 * kk) : u32x4_t{0, 0, 0, 0};
                vr[p][kk] = live ? *reinterpret_cast<const u32x4_t *>(a.v_cache + base + 32 * kk) : u32x4_t{0, 0, 0, 0};
            }
        }
    };

    f32x4_t oacc[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, lsum = 0.f;

    uint16_t *slab = reinterpret_cast<uint16_t *>(smem_raw) + wave * SM::slab;

    int st = wave;
    if (st < nsteps) load_step(st, kc, vc, bad);
    for (; st < nsteps; st += kWaves) {
        u32x4_t kn[2][D / 32], vn[2][D / 32];
        const bool more = st + kWaves < nsteps;
        if (more) load_step(st + kWaves, kn, vn, bad);

        // S^T (16 tokens x 16 heads) per block.
        f32x4_t s[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            s[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) s[p] = mfma_16x16x32_bf16(kc[p][kk], qf[kk], s[p]);
        }
        // Lane (g, l16) holds tokens 4g + v of each block for head l16.
        float mx = kNegInf;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = (blk0 + 2 * st + p) * kBS + 4 * g + v;
                const float t = tok < t_end ? s[p][v] * a.scale_log2 : kNegInf;
                s[p][v] = t;
                mx = fmaxf(mx, t);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        const bool grow = m_new > m + 8.0f;
        if (wave_any(grow)) {
            const float alpha = grow ? exp2_fast(m - m_new) : 1.0f;
            m = grow ? m_new : m;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
        }
        const float mref = (m == kNegInf) ? 0.f : m;
        float pv[2][4];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                pv[p][v] = exp2_fast(s[p][v] - mref);
                lsum += pv[p][v];
            }
        // P^T operand: k-slots 0..3 = block 0 tokens 4g..4g+3, 4..7 = block 1.
        const u32x4_t pk = {pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                            pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])};

        // V^T operand through LDS: write both blocks row-major, read columns.
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                *reinterpret_cast<u32x4_t *>(slab + (p * kBS + l16) * SM::pitch + 32 * kk + 8 * g) = vc[p][kk];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            const uint16_t *col = slab + 4 * g * SM::pitch + 16 * db + l16;
            u32x4_t a_op;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int p = e >> 1, r = 2 * (e & 1);
                const uint32_t x0 = col[(p * kBS + r) * SM::pitch];
                const uint32_t x1 = col[(p * kBS + r + 1) * SM::pitch];
                a_op[e] = x0 | (x1 << 16);
            }
            oacc[db] = mfma_16x16x32_bf16(a_op, pk, oacc[db]);
        }
        __builtin_amdgcn_wave_barrier();

        if (more) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int kk = 0; kk < D / 32; ++kk) {
                    kc[p][kk] = kn[p][kk];
                    vc[p][kk] = vn[p][kk];
                }
        }
    }

    // Row sums: lanes g = 0..3 of a head hold disjoint tokens.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    // Merge the four wave partials of this chunk in LDS.
    __syncthreads();                                    // V slabs are free now
    float *cm = reinterpret_cast<float *>(smem_raw);    // [wave][16] m, then l, then O [wave][16][D]
    float *cl = cm + kWaves * 16;
    float *co = cl + kWaves * 16;
    if (g == 0) {
        cm[wave * 16 + l16] = m;
        cl[wave * 16 + l16] = lsum;
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int v = 0; v < 4; ++v) co[(wave * 16 + l16) * D + 16 * db + 4 * g + v] = oacc[db][v];
    const bool any_bad = __syncthreads_or(bad);

    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int head = idx / D, d = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, cm[w * 16 + head]);
        float L = 0.f, O = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = cm[w * 16 + head];
                if (mw == kNegInf) continue;
                const float sc = exp2_fast(mw - M);
                L += cl[w * 16 + head] * sc;
                O += co[(w * 16 + head) * D + d] * sc;
            }
        }
        const size_t row = ((size_t)b * a.Hq + hk * G + head) * a.splits + split;
        float o_out = L > 0.f ? O / L : 0.f;
        float lse_out = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
        if (any_bad) {
            o_out = __builtin_nanf("");
            lse_out = __builtin_nanf("");
        }
        a.part_o[row * D + d] = o_out;
        if (d == 0) a.part_lse[row] = lse_out;
    }
}

// One wave per (sequence, query head).
template <int D>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeArgs a)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // b * Hq + hq
    if (row >= a.B * a.Hq) return;
    constexpr int PER = D / 64;                            // d values per lane
    const float *plse = a.part_lse + (size_t)row * a.splits;
    const float *po = a.part_o + (size_t)row * a.splits * D;

    float M = kNegInf;
    bool nan = false;
    for (int s = 0; s < a.splits; ++s) {
        const float x = plse[s];
        nan |= (x != x);
        M = fmaxf(M, x);
    }
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    float wsum = 0.f;
    if (M != kNegInf && !nan) {
        for (int s = 0; s < a.splits; ++s) {
            const float x = plse[s];
            if (x == kNegInf) continue;
            const float w = exp2_fast((x - M) * kLog2e);
            wsum += w;
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] += w * po[(size_t)s * D + lane + 64 * i];
        }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    uint16_t *op = a.o + (size_t)row * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const float val = nan ? __builtin_nanf("") : acc[i] * inv;
        const uint32_t packed = pack_bf16x2(val, 0.f);
        op[lane + 64 * i] = (uint16_t)(packed & 0xFFFFu);
    }
    if (a.lse != nullptr && lane == 0)
        a.lse[row] = nan ? __builtin_nanf("") : (wsum > 0.f ? M + logf(wsum) : kNegInf);
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s)
{
    const long long g1 = (long long)a.B * a.Hkv * a.splits;
    if (g1 <= 0) return hipSuccess;
    hipLaunchKernelGGL((decode_split_kernel<D>), dim3((unsigned)g1), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long g2 = ((long long)a.B * a.Hq + 3) / 4;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)g2), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int head_dim, hipStream_t s)
{
    if (head_dim == 128) return launch_d<128>(a, s);
    if (head_dim == 64) return launch_d<64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
