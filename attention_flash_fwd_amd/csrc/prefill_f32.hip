// prefill_f32.hip -- exact attention forward with fp32 inputs, outputs and
// arithmetic throughout (no bf16 rounding anywhere), on the fp32 matrix-core
// form v_mfma_f32_32x32x2_f32.
//
// Same FlashAttention structure as the bf16 kernel ("推理加速" interview notes,
// section FlashAttention; chenyy20.com "抱infra脚", Flash Attention 基本原理 /
// 核心技术): a workgroup owns 128 query rows (4 waves x 32), K/V tiles of 64
// keys are staged in LDS, S^T = K Q^T leaves one query row per lane, the
// online softmax keeps a running max and sum, and O^T += V^T P^T takes P
// straight from the score registers.  This path exists for exactness, not
// speed: it stages through LDS with a single buffer and scalar LDS accesses.
#include "gfx950.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kBR = 128;
constexpr int kBC = 64;
constexpr int kThreads = 256;

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) prefill_f32_kernel(PrefillArgs a)
{
    constexpr int P = D + 1;   // LDS row pitch in floats: consecutive rows start in consecutive banks
    __shared__ float ks[kBC * P];
    __shared__ float vs[kBC * P];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;

    const int n_qtiles = (a.Sq + kBR - 1) / kBR;
    const int qt = n_qtiles - 1 - (int)(blockIdx.x % n_qtiles);
    const int bh = blockIdx.x / n_qtiles;
    const int b = bh / a.Hq, hq = bh % a.Hq;
    const int G = a.Hq / a.Hkv, hk = hq / G;
    const int i0 = qt * kBR;
    const int q0 = i0 + wave * 32;
    const int my_q = q0 + l32;
    const int diag = a.Sk - a.Sq;

    int kend = a.Sk;
    if (CAUSAL) kend = min(a.Sk, min(a.Sq, i0 + kBR) + diag);
    const int ntiles = kend > 0 ? (kend + kBC - 1) / kBC : 0;

    const float *qg = static_cast<const float *>(a.q);
    const size_t kv_rs = (size_t)a.Hkv * D;
    const float *kbase = static_cast<const float *>(a.k) + (size_t)b * a.Sk * kv_rs + (size_t)hk * D;
    const float *vbase = static_cast<const float *>(a.v) + (size_t)b * a.Sk * kv_rs + (size_t)hk * D;

    // Q^T operand: lane (h, l32) holds q[my_q][2 ks + h].
    float qf[D / 2];
    {
        const float *qp = qg + (((size_t)b * a.Sq + my_q) * a.Hq + hq) * D;
#pragma unroll
        for (int ks2 = 0; ks2 < D / 2; ++ks2) qf[ks2] = my_q < a.Sq ? qp[2 * ks2 + h] : 0.f;
    }

    f32x16_t oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m = kNegInf, lsum = 0.f;

    for (int j = 0; j < ntiles; ++j) {
        const int kv0 = j * kBC;
        // Stage the tile; keys past the end are zero so masked P*V stays 0.
        for (int e = tid; e < kBC * D; e += kThreads) {
            const int row = e / D, col = e % D;
            const int key = kv0 + row;
            ks[row * P + col] = key < a.Sk ? kbase[key * kv_rs + col] : 0.f;
            vs[row * P + col] = key < a.Sk ? vbase[key * kv_rs + col] : 0.f;
        }
        __syncthreads();

        bool live[2];
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int kstart = kv0 + 32 * kb;
            live[kb] = kstart < a.Sk && (!CAUSAL || kstart <= q0 + 31 + diag);
#pragma unroll
            for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
            if (live[kb]) {
                const float *kr = ks + (32 * kb + l32) * P + h;
#pragma unroll
                for (int ks2 = 0; ks2 < D / 2; ++ks2) s[kb] = mfma_32x32x2_f32(kr[2 * ks2], qf[ks2], s[kb]);
            }
        }

        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = kv0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
                const bool vis = key < a.Sk && (!CAUSAL || key <= my_q + diag);
                const float t = vis ? s[kb][v] * a.scale_log2 : kNegInf;
                s[kb][v] = t;
                mx = fmaxf(mx, t);
            }
        }
        mx = pair_max_halves(mx);
        const float m_new = fmaxf(m, mx);
        if (m_new > m) {
            const float alpha = exp2_fast(m - m_new);
            m = m_new;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
        }
        const float mref = (m == kNegInf) ? 0.f : m;

#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = exp2_fast(s[kb][v] - mref);
                lsum += p;
                s[kb][v] = p;
            }
            if (!live[kb]) continue;
            // k-slot h of MFMA v pairs key 32kb + 8(v/4) + 4h + v%4 with P from this lane.
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float *vr = vs + (32 * kb + 8 * (v >> 2) + 4 * h + (v & 3)) * P + l32;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) oacc[db] = mfma_32x32x2_f32(vr[32 * db], s[kb][v], oacc[db]);
            }
        }
        __syncthreads();
    }

    const float ltot = pair_sum_halves(lsum);
    if (my_q < a.Sq) {
        const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
        float *op = static_cast<float *>(a.o) + (((size_t)b * a.Sq + my_q) * a.Hq + hq) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4_t w = {oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                                   oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
                *reinterpret_cast<f32x4_t *>(op + 32 * db + 8 * g4 + 4 * h) = w;
            }
        if (a.lse != nullptr && h == 0)
            a.lse[((size_t)b * a.Hq + hq) * a.Sq + my_q] = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : kNegInf;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s)
{
    const int n_qtiles = (a.Sq + kBR - 1) / kBR;
    const long long grid = (long long)n_qtiles * a.Hq * a.B;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs &a, int head_dim, bool causal, hipStream_t s)
{
    if (head_dim == 128) return causal ? launch_one<128, true>(a, s) : launch_one<128, false>(a, s);
    if (head_dim == 64) return causal ? launch_one<64, true>(a, s) : launch_one<64, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
