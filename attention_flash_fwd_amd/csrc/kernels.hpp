// kernels.hpp -- argument blocks and launchers of the device kernels.
// Host code (attn_api.cpp) validates every argument before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct PrefillArgs {
    const void *q, *k, *v;    // [B,Sq,Hq,D], [B,Sk,Hkv,D], [B,Sk,Hkv,D]
                              // (paged: k, v are caches [num_blocks,16,Hkv,D])
    void *o;                  // [B,Sq,Hq,D]
    float *lse;               // [B,Hq,Sq] or nullptr
    int B, Sq, Sk, Hq, Hkv;   // paged: Sk unused, keys per sequence in ctx_lens
    float scale_log2;         // softmax scale times log2(e)
    // Paged keys and values only:
    const int32_t *block_table;   // [B,max_blocks]
    const int32_t *ctx_lens;      // [B]
    int num_blocks, max_blocks;
};

struct DecodeArgs {
    const uint16_t *q;            // [B,T,Hq,D] bf16 (T new tokens per sequence)
    const void *k_cache;          // [num_blocks,16,Hkv,D] bf16 or fp8 e4m3
    const void *v_cache;
    const int32_t *block_table;   // [B,max_blocks]
    const int32_t *ctx_lens;      // [B]
    float *part_o;                // [B,T,Hq,splits,D] fp32
    float *part_lse;              // [B,T,Hq,splits]   fp32
    uint16_t *o;                  // [B,T,Hq,D] bf16
    float *lse;                   // [B,Hq,T] or nullptr
    int B, T, Hq, Hkv, num_blocks, max_blocks, splits;
    float scale_log2;             // softmax scale (times the K dequantisation scale) times log2(e)
    float v_scale;                // V dequantisation scale (1 for bf16 caches)
    unsigned *work_ctr;           // split-kernel work counter in the workspace (zeroed by the launch)
};

// Compute units of the current device (cached per device).
int compute_units();

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, bool causal, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs &a, int head_dim, bool causal, hipStream_t s);
hipError_t launch_prefill_paged_bf16(const PrefillArgs &a, int head_dim, bool causal, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int head_dim, bool kv_fp8, hipStream_t s);
// Split kernel for many (token, head) columns (more than 32 over a bf16
// cache, more than 64 over an e4m3 cache at head_dim 128), writing the
// partials as launch_decode's split kernel does (no merge).
bool decode_wide_supported(int head_dim, bool kv_fp8, long long columns);
hipError_t launch_decode_wide(const DecodeArgs &a, int head_dim, bool kv_fp8, hipStream_t s);

// Device address of the library-held decode workspace of the current device
// (ATTN_STATIC_SCRATCH_BYTES bytes; looked up once per device), or nullptr if
// the lookup failed.
void *static_scratch();

}  // namespace attn
