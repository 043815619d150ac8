// hbm_probe.hip -- libgqa_probe.so: plain streaming kernels that measure the
// practical HBM bandwidth of the GPU, as a ceiling to compare the decode
// kernels against. Not part of the attention library; only the benchmark
// loads it.
//
//   gqa_probe_read(buf, bytes, nontemporal, sink, stream): every byte of buf
//     is read once with 16-byte loads; each thread folds what it read into
//     one word written to sink[thread] so the loads cannot be dropped.
//   gqa_probe_copy(dst, src, bytes, stream): dst = src with 16-byte loads and
//     stores.
// bytes must be a multiple of 16 * 4096, pointers 16-byte aligned; sink holds
// kProbeThreads words.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kBlocks = 2048;  // 8 workgroups per compute unit
constexpr int kThreads = 256;

template <bool NT>
__global__ void __launch_bounds__(kThreads) probe_read_kernel(const probe_u32x4 *__restrict__ src, int64_t n16,
                                                              uint32_t *__restrict__ sink)
{
    // Each workgroup streams one contiguous slice, four loads in flight per thread.
    const int64_t per = n16 / gridDim.x;
    const probe_u32x4 *p = src + (int64_t)blockIdx.x * per;
    uint32_t acc = 0;
    for (int64_t i = threadIdx.x; i < per; i += 4 * kThreads) {
        probe_u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = i + u * kThreads;
            const probe_u32x4 *a = p + (j < per ? j : per - 1);
            v[u] = NT ? __builtin_nontemporal_load(a) : *a;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ void __launch_bounds__(kThreads) probe_copy_kernel(probe_u32x4 *__restrict__ dst,
                                                              const probe_u32x4 *__restrict__ src, int64_t n16)
{
    const int64_t per = n16 / gridDim.x;
    const int64_t base = (int64_t)blockIdx.x * per;
    for (int64_t i = threadIdx.x; i < per; i += 4 * kThreads) {
        probe_u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = i + u * kThreads;
            v[u] = __builtin_nontemporal_load(src + base + (j < per ? j : per - 1));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = i + u * kThreads;
            if (j < per)
                __builtin_nontemporal_store(v[u], dst + base + j);
        }
    }
}

}  // namespace

extern "C" {

int gqa_probe_threads(void)
{
    return kBlocks * kThreads;
}

// 0 on success, else the HIP error code (1 for bad arguments).
int gqa_probe_read(const void *buf, int64_t bytes, int nontemporal, uint32_t *sink, hipStream_t stream)
{
    if (!buf || !sink || bytes <= 0 || bytes % (16 * kBlocks) != 0 || (reinterpret_cast<uintptr_t>(buf) & 15))
        return 1;
    const int64_t n16 = bytes / 16;
    if (nontemporal)
        probe_read_kernel<true><<<kBlocks, kThreads, 0, stream>>>(static_cast<const probe_u32x4 *>(buf), n16, sink);
    else
        probe_read_kernel<false><<<kBlocks, kThreads, 0, stream>>>(static_cast<const probe_u32x4 *>(buf), n16, sink);
    return (int)hipGetLastError();
}

int gqa_probe_copy(void *dst, const void *src, int64_t bytes, hipStream_t stream)
{
    if (!dst || !src || bytes <= 0 || bytes % (16 * kBlocks) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) ||
        (reinterpret_cast<uintptr_t>(src) & 15))
        return 1;
    probe_copy_kernel<<<kBlocks, kThreads, 0, stream>>>(static_cast<probe_u32x4 *>(dst),
                                                       static_cast<const probe_u32x4 *>(src), bytes / 16);
    return (int)hipGetLastError();
}

}  // extern "C"
