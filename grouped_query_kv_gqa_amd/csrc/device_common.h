// device_common.h -- small gfx950 helpers shared by the libgqa kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define GQA_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace gqa {

constexpr float kLog2e = 1.4426950408889634f;

// 16x16x32 bf16 MFMA, fp32 accumulate. Lane l supplies A[l%16][8*(l/16) .. +7]
// and B[8*(l/16) .. +7][l%16]; it receives C[4*(l/16) .. +3][l%16].
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 32x32x16 bf16 MFMA, fp32 accumulate. Lane l supplies A[l%32][8*(l/32) .. +7]
// and B[8*(l/32) .. +7][l%32]; register v = 4*m0 + m1 of the result holds
// C[8*m0 + 4*(l/32) + m1][l%32].
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i addresses 4 consecutive 16-bit elements at row i/4, columns
// 4*(i%4) .. +3 of a 4 x 16 block; after the read lane i holds column i of
// that block, rows 0..3.
__device__ __forceinline__ bf16x4_t lds_read_tr16(const __bf16 *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GQA_LDS bf16x4_t *)(p));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// Two floats to two bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8_t pack_bf16x8(f32x4_t a, f32x4_t b)
{
    u32x4_t u;
    u[0] = pack_bf16x2(a[0], a[1]);
    u[1] = pack_bf16x2(a[2], a[3]);
    u[2] = pack_bf16x2(b[0], b[1]);
    u[3] = pack_bf16x2(b[2], b[3]);
    return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ float fast_exp2(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float fast_log2(float x)
{
    return __builtin_amdgcn_logf(x);
}

__device__ __forceinline__ float wave_max_xor(float x, int mask)
{
    return fmaxf(x, __shfl_xor(x, mask, 64));
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}

__device__ __forceinline__ int clamp_len(int32_t L, int Tmax)
{
    return L < 0 ? 0 : (L > Tmax ? Tmax : (int)L);
}

// Wait until every vector memory operation this wave issued has completed
// (stores acknowledged): s_waitcnt vmcnt(0) with expcnt and lgkmcnt left free.
__device__ __forceinline__ void wait_vector_memory()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Compiler-level ordering point for memory operations of one wave.
__device__ __forceinline__ void compiler_fence()
{
    asm volatile("" ::: "memory");
}

}  // namespace gqa
