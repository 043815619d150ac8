// prefill.hip -- GQA prefill (every position of a sequence is a query).
//
// out[b,t,h,:] = sum_{s in keys(t)} softmax_s(q[b,t,h,:] . k[b,s,g,:] / sqrt(d_h)) v[b,s,g,:]
// with g = h / r and keys(t) = [0, t] when causal, [0, T) otherwise
// ("Grouped-Query Attention" (llm-arch-kb), section 3 Reference
// implementation: broadcast of each key/value head to its H/G query heads,
// scores over sqrt(d_h), causal mask, softmax over keys, times v).
//
// Row kernel: one wavefront per (b, t, h) row, lanes split d_h, online
// softmax over the keys one position at a time, fp32 arithmetic.
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T *p);
template <>
__device__ __forceinline__ float ld<float>(const float *p)
{
    return *p;
}
template <>
__device__ __forceinline__ float ld<__bf16>(const __bf16 *p)
{
    return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(p));
}

template <typename T>
__device__ __forceinline__ void st(T *p, float x);
template <>
__device__ __forceinline__ void st<float>(float *p, float x)
{
    *p = x;
}
template <>
__device__ __forceinline__ void st<__bf16>(__bf16 *p, float x)
{
    *reinterpret_cast<uint16_t *>(p) = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}

template <typename T, int D>
__global__ void __launch_bounds__(64)
prefill_row_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, int T_, int H,
                   int G, int causal, float scale, T *__restrict__ out)
{
    constexpr int J = D / 64;
    const int64_t row = blockIdx.x;  // ((b * T) + t) * H + h
    const int h = (int)(row % H);
    const int64_t bt = row / H;
    const int t = (int)(bt % T_);
    const int64_t b = bt / T_;
    const int r = H / G;
    const int g = h / r;
    const int lane = threadIdx.x;
    const int nkeys = causal ? t + 1 : T_;
    float qv[J], acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        qv[j] = ld(q + row * D + lane + 64 * j);
        acc[j] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int s = 0; s < nkeys; ++s) {
        const int64_t off = ((b * T_ + s) * G + g) * D;
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j)
            dot += qv[j] * ld(k + off + lane + 64 * j);
        const float sc = wave_sum(dot) * scale;
        const float m_new = fmaxf(m, sc);
        const float alpha = expf(m - m_new);
        const float p = expf(sc - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int j = 0; j < J; ++j)
            acc[j] = acc[j] * alpha + p * ld(v + off + lane + 64 * j);
        m = m_new;
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
        st(out + row * D + lane + 64 * j, acc[j] / l);
}

template <typename T>
hipError_t launch_rows(const PrefillArgs &a)
{
    const int64_t rows = (int64_t)a.B * a.T * a.H;
    const float scale = 1.0f / sqrtf((float)a.D);
    if (a.D == 64)
        prefill_row_kernel<T, 64><<<dim3((unsigned)rows), 64, 0, a.stream>>>(
            static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v), a.T, a.H, a.G,
            a.causal, scale, static_cast<T *>(a.out));
    else
        prefill_row_kernel<T, 128><<<dim3((unsigned)rows), 64, 0, a.stream>>>(
            static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v), a.T, a.H, a.G,
            a.causal, scale, static_cast<T *>(a.out));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, gqa_dtype dtype)
{
    if (dtype == GQA_FP32)
        return launch_rows<float>(a);
    return launch_rows<__bf16>(a);
}

}  // namespace gqa
