// hbm_probe.hip -- libgqa_probe.so: plain streaming kernels that measure the
// practical HBM bandwidth of the GPU, as a ceiling to compare the decode
// kernels against. Not part of the attention library; only the benchmark
// loads it.
//
//   gqa_probe_read(buf, bytes, nontemporal, sink, stream): every byte of buf
//     is read once with 16-byte loads; each thread folds what it read into
//     one word written to sink[thread] so the loads cannot be dropped.
//   gqa_probe_read_wide(buf, bytes, sink, stream): the same read by one
//     8-wave workgroup per compute unit, each streaming one contiguous slice
//     in rounds of 16 nontemporal 16-byte loads per thread (128 KiB per
//     workgroup) issued together and then consumed: on this chip the faster
//     of the two reads.
//   gqa_probe_copy(dst, src, bytes, stream): dst = src with 16-byte loads and
//     stores.
// bytes must be a multiple of 16 * 2048 (16 * 256 for the wide read),
// pointers 16-byte aligned; sink holds gqa_probe_threads() words.
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

constexpr int kWideBlocks = 256;  // one per compute unit
constexpr int kWideThreads = 512;
constexpr int kWideLoads = 16;    // loads in flight per thread

__global__ void __launch_bounds__(kWideThreads) probe_read_wide_kernel(const probe_u32x4 *__restrict__ src,
                                                                       int64_t n16, uint32_t *__restrict__ sink)
{
    const int64_t per = n16 / gridDim.x;
    const probe_u32x4 *p = src + (int64_t)blockIdx.x * per;
    uint32_t acc = 0;
    for (int64_t i = threadIdx.x; i < per; i += kWideLoads * kWideThreads) {
        probe_u32x4 v[kWideLoads];
#pragma unroll
        for (int u = 0; u < kWideLoads; ++u) {
            const int64_t j = i + u * kWideThreads;
            v[u] = __builtin_nontemporal_load(p + (j < per ? j : per - 1));
        }
        // keep the round's loads together: without the fence the compiler
        // interleaves each load with its use
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kWideLoads; ++u)
            acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
    sink[(int64_t)blockIdx.x * kWideThreads + threadIdx.x] = acc;
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

int gqa_probe_read_wide(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (!buf || !sink || bytes <= 0 || bytes % (16 * kWideBlocks) != 0 || (reinterpret_cast<uintptr_t>(buf) & 15))
        return 1;
    static_assert(kWideBlocks * kWideThreads <= kBlocks * kThreads, "the sink holds one word per thread");
    probe_read_wide_kernel<<<kWideBlocks, kWideThreads, 0, stream>>>(static_cast<const probe_u32x4 *>(buf),
                                                                       bytes / 16, sink);
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
