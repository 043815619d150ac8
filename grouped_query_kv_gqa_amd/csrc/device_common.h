// device_common.h -- small gfx950 helpers shared by the libgqa kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#define GQA_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

namespace gqa {

constexpr float kLog2e = 1.4426950408889634f;

// A compile-time integer as a type (selects LDS buffers statically).
template <int I>
using Ic = std::integral_constant<int, I>;

// The 16-bit kernels are templates over the storage type T (__bf16 or
// _Float16). Registers and LDS hold the raw 16-bit patterns in bf16x8_t /
// bf16x4_t containers for either type; the helpers below pick the matching
// MFMA and conversion instructions.
template <typename T>
inline constexpr bool kIsF16 = __is_same(T, _Float16);

// 16x16x32 MFMA, fp32 accumulate. Lane l supplies A[l%16][8*(l/16) .. +7]
// and B[8*(l/16) .. +7][l%16]; it receives C[4*(l/16) .. +3][l%16].
template <typename T>
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    if constexpr (kIsF16<T>)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 32x32x16 MFMA, fp32 accumulate. Lane l supplies A[l%32][8*(l/32) .. +7]
// and B[8*(l/32) .. +7][l%32]; register v = 4*m0 + m1 of the result holds
// C[8*m0 + 4*(l/32) + m1][l%32].
template <typename T>
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    if constexpr (kIsF16<T>)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i addresses 4 consecutive 16-bit elements at row i/4, columns
// 4*(i%4) .. +3 of a 4 x 16 block; after the read lane i holds column i of
// that block, rows 0..3. It moves bits only, so it serves either 16-bit type.
__device__ __forceinline__ bf16x4_t lds_read_tr16(const __bf16 *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GQA_LDS bf16x4_t *)(p));
}

// The value of one stored 16-bit pattern (low 16 bits of bits16).
template <typename T>
__device__ __forceinline__ float bits_to_f32(uint32_t bits16)
{
    if constexpr (kIsF16<T>)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
    else
        return __uint_as_float(bits16 << 16);
}

// Two floats to two T, round to nearest even (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32), lo in the low half.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    if constexpr (kIsF16<T>)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

template <typename T>
__device__ __forceinline__ bf16x8_t pack8(f32x4_t a, f32x4_t b)
{
    u32x4_t u;
    u[0] = pack2<T>(a[0], a[1]);
    u[1] = pack2<T>(a[2], a[3]);
    u[2] = pack2<T>(b[0], b[1]);
    u[3] = pack2<T>(b[2], b[3]);
    return __builtin_bit_cast(bf16x8_t, u);
}

// acc + (sum of the two T values packed in w), one dot-product instruction.
template <typename T>
__device__ __forceinline__ float add_pair(uint32_t w, float acc)
{
    if constexpr (kIsF16<T>)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), (f16x2_t){(_Float16)1.f, (_Float16)1.f}, acc,
                                      false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), (bf16x2_t){(__bf16)1.f, (__bf16)1.f},
                                               acc, false);
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

// x of this lane and of lane l ^ MASK, exchanged on the VALU: for MASK = 16
// or 32 by the lane swaps (v_permlane16_swap / v_permlane32_swap with both
// operands x), for MASK = 1, 2, 4 or 8 by DPP moves within rows of 16 lanes
// (quad_perm for 1 and 2, row_ror:8 for 8, row_shl:4 or row_shr:4 by lane
// for 4). `a`, `b` are the two values, in an order that may differ between
// the two lanes of a pair, so their maximum or sum is the same in both
// lanes. Unlike __shfl_xor (ds_bpermute) no exchange goes through the LDS
// queue or waits behind outstanding LDS reads. Lane layout checked on
// gfx950. The swap results are copied to scalars before the bit casts:
// clang's __builtin_bit_cast of a vector element expression reads the
// vector's first element whatever the index.
template <int MASK>
__device__ __forceinline__ void xor_pair(float x, float &a, float &b)
{
    static_assert(MASK == 1 || MASK == 2 || MASK == 4 || MASK == 8 || MASK == 16 || MASK == 32,
                  "lane exchanges for xor masks 1 to 32");
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    if constexpr (MASK >= 16) {
        uint32_t s0, s1;
        if constexpr (MASK == 32) {
            const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            s0 = s[0];
            s1 = s[1];
        } else {
            const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
            s0 = s[0];
            s1 = s[1];
        }
        a = __builtin_bit_cast(float, s0);
        b = __builtin_bit_cast(float, s1);
    } else {
        const int v = (int)u;
        int p;
        if constexpr (MASK == 1) {
            p = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
        } else if constexpr (MASK == 2) {
            p = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
        } else if constexpr (MASK == 8) {
            p = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
        } else {
            const int up = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);    // row_shl:4: lane + 4
            const int down = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4: lane - 4
            p = (__lane_id() & 4) ? down : up;
        }
        a = x;
        b = __builtin_bit_cast(float, p);
    }
}

template <int MASK>
__device__ __forceinline__ float xor_fmax(float x)
{
    float a, b;
    xor_pair<MASK>(x, a, b);
    return fmaxf(a, b);
}

template <int MASK>
__device__ __forceinline__ float xor_add(float x)
{
    float a, b;
    xor_pair<MASK>(x, a, b);
    return a + b;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}

__device__ __forceinline__ double wave_sum(double x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips): within each row of 16 lanes by shifts
// of 1, 2, 4 and 8, then row 0's total into row 1, row 2's into row 3, and
// lane 31's running total into rows 2 and 3. Lanes whose DPP source is
// outside the row or whose row is masked add the `old` operand, 0.
__device__ __forceinline__ int wave_incl_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return x;
}

// Sum over the wave, the same in every lane (wave-uniform).
__device__ __forceinline__ int wave_total(int x)
{
    return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

__device__ __forceinline__ int clamp_len(int32_t L, int Tmax)
{
    return L < 0 ? 0 : (L > Tmax ? Tmax : (int)L);
}

// N buffer_load_dwordx4 ... lds from a raw buffer of nrec bytes at base:
// instruction u reads byte voff + u*step of the buffer (zeros past nrec) into
// LDS at dst + u*dst_step elements, lane i at +16*i bytes. The whole byte
// offset goes in the per-lane (vector) offset: for a raw buffer the range
// check compares only the vector plus instruction offset with nrec, and a
// part carried in the scalar offset would be added after the check, so rows
// past the end would be read instead of returning zeros.
// CPOL selects the cache policy (0: default; kCpolNT: nontemporal, for rows
// read once).
constexpr int kCpolNT = 2;

template <int N, int CPOL = 0>
__device__ __forceinline__ void buffer_rows_to_lds(const __bf16 *base, int nrec, __bf16 *dst, int dst_step, int voff,
                                                   int step)
{
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16 *>(base), (short)0, nrec, 0x00020000);
#pragma unroll
    for (int u = 0; u < N; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (GQA_LDS void *)(dst + u * dst_step), 16, voff + u * step, 0,
                                                 0, CPOL);
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

// Debug builds (-DGQA_DEBUG): range checks at the kernels' global memory
// accesses. A failed check sets bit `site` of this source file's violation
// word and the access is skipped (a load gives zeros), so an indexing
// mistake shows up as a flag that the host reads back (gqa_debug_checks)
// instead of as a memory fault. Release builds compile the checks away.
// Each source file that includes this header has its own word and defines
// its reader with GQA_DEBUG_READER(name).
#ifdef GQA_DEBUG
static __device__ unsigned int gqa_debug_word;

__device__ __forceinline__ bool debug_in_range(int64_t i, int64_t n, int site)
{
    if (i >= 0 && i < n)
        return true;
    atomicOr(&gqa_debug_word, 1u << site);
    return false;
}

#define GQA_IN_RANGE(i, n, site) ::gqa::debug_in_range((int64_t)(i), (int64_t)(n), (site))
// Host reader: copies this file's word to *w and clears it (synchronous).
#define GQA_DEBUG_READER(name)                                                                 \
    hipError_t name(unsigned int *w)                                                           \
    {                                                                                          \
        hipError_t e = hipMemcpyFromSymbol(w, HIP_SYMBOL(gqa_debug_word), sizeof(unsigned int)); \
        if (e != hipSuccess)                                                                   \
            return e;                                                                          \
        const unsigned int zero = 0;                                                           \
        return hipMemcpyToSymbol(HIP_SYMBOL(gqa_debug_word), &zero, sizeof zero);              \
    }
#else
#define GQA_IN_RANGE(i, n, site) true
#define GQA_DEBUG_READER(name)        \
    hipError_t name(unsigned int *w)  \
    {                                 \
        *w = 0;                       \
        return hipSuccess;            \
    }
#endif

}  // namespace gqa
