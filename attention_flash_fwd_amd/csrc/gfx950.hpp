// gfx950.hpp -- CDNA4 (MI355X, gfx950) building blocks shared by the kernels:
// matrix-core (MFMA) wrappers with their register layouts, wave-half
// exchanges, exp2 and bf16 packing.
//
// Register layouts of the MFMA forms used here (wave64, lane l):
//   v_mfma_f32_32x32x16_bf16  A: row l%32, 8 k-values   (k-slots 8*(l/32)..+7)
//                             B: col l%32, 8 k-values   (same k-slot mapping)
//                             C: col l%32, 16 rows 8*(v/4) + 4*(l/32) + v%4
//   v_mfma_f32_16x16x32_bf16  A: row l%16, 8 k-values   (k-slots 8*(l/16)..+7)
//                             B: col l%16, 8 k-values
//                             C: col l%16, 4 rows 4*(l/16) + v
//   v_mfma_f32_32x32x2_f32    A: row l%32, k-slot l/32;  B: col l%32, k-slot l/32
//                             C: as for 32x32x16.
// A contraction only needs A and B to agree on which k each (lane, element)
// slot carries, so callers are free to permute the contraction index (the
// kernels use that to chain the score accumulator straight into the PV
// operand without a trip through LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16_t mfma_32x32x16_bf16(u32x4_t a, u32x4_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_32x32x2_f32(float a, float b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32);
// a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// Four e4m3 values (one word, value i in byte i) -> four bf16 in two words,
// with v_cvt_scalef32_pk_bf16_fp8 at scale 1.0 (exact: every e4m3 value is
// a bf16 value).
__device__ __forceinline__ u32x2_t fp8x4_to_bf16(uint32_t x)
{
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
    return u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Combine a value with the one held by the lane 32 positions away
// (v_permlane32_swap: the two wave halves trade their copies), returning
// max / sum over the pair in every lane.
__device__ __forceinline__ float pair_max_halves(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Max with the value held by the lane 16 positions away within each half
// of the wave (v_permlane16_swap: lanes 16-31 and 0-15, and 48-63 and 32-47,
// trade their copies), in every lane.
__device__ __forceinline__ float pair_max_quarters(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum_halves(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Byte permute (v_perm_b32): bytes 0-3 come from lo, 4-7 from hi.
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low 16-bit halves of two words: lo16(a) | lo16(b) << 16.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return byte_perm(b, a, 0x05040100u); }
// High 16-bit halves of two words: hi16(a) | hi16(b) << 16.
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return byte_perm(b, a, 0x07060302u); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Values the compiler cannot prove wave-uniform but that are: move them to
// scalar registers so that buffer descriptors and LDS bases stay scalar.
// (readfirstlane returns a signed int: go through uint32_t so that nothing
// is sign-extended into the upper address bits.)
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ void *uniform_ptr(const void *p)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = uniform_u32((uint32_t)a);
    const uint64_t hi = uniform_u32((uint32_t)(a >> 32));
    return reinterpret_cast<void *>(lo | (hi << 32));
}

// Returns x unchanged but hides its value from the optimiser, so that
// per-lane address arithmetic derived from it stays where it is written
// instead of being hoisted out of a loop into long-lived registers.
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// Raw buffer descriptor over [base, base + bytes): loads at offsets past the
// end return zero (word 3 = 0x00020000, the gfx9 raw-buffer format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base), (short)0, (int)uniform_u32(bytes), 0x00020000);
}

// 16 bytes per lane from buffer offset voff (zero past the end of the buffer).
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses
// but leaves its global loads in flight (a full __syncthreads() fence would
// also wait for every outstanding global load).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 16 bytes per lane from buffer offset voff straight into LDS: the wave's 64
// lanes fill the 1 KiB at lds (lane i at lds + 16 i).  Completion is tracked
// by vmcnt like any vector-memory load.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte words read by lanes
// i / 4 + 4 e (e = 0..3) of its group.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t *p)
{
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t *)(p));
    return __builtin_bit_cast(u32x2_t, r);
}

}  // namespace attn
