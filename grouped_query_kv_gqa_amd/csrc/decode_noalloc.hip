// decode_noalloc.hip -- gqa_decode_step_noalloc: the decode step with its
// split workspace (fp32 partial rows and their log-sum-exp values) in a
// fixed device array of this library instead of allocated memory, for
// callers that cannot allocate (graph capture, tight serving loops).
//
// The array is file-scope device memory: the code object holds one copy per
// GPU it is loaded on, kept until the process ends. Host code must not pass
// the array's name to a kernel (on the host it names a stand-in, not device
// memory): its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// used. Every call on a GPU shares that GPU's array, so calls that overlap
// in time on one GPU (on different streams, or graph replays running
// concurrently with them) race on it. Nothing in it needs clearing between
// calls: every slot the merge kernel reads was written earlier in the same
// call.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <unordered_map>

#include "api_internal.h"
#include "gqa.h"

static constexpr int64_t kScratchBytes = int64_t(32) << 20;  // 32 MiB per GPU

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mutex;
std::unordered_map<int, char *> g_scratch_ptr;  // device -> device address of `scratch`

// The device address of `scratch` on the current device (looked up once).
gqa_status scratch_on_current_device(char **out)
{
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return gqa::set_last_error(GQA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    auto it = g_scratch_ptr.find(device);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return GQA_OK;
    }
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
        return gqa::set_last_error(GQA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                                    hipGetErrorString(e != hipSuccess ? e : hipErrorInvalidSymbol));
    g_scratch_ptr[device] = static_cast<char *>(ptr);
    *out = static_cast<char *>(ptr);
    return GQA_OK;
}

}  // namespace

extern "C" gqa_status gqa_decode_step_noalloc(const void *q, const void *k_new, const void *v_new, void *k_cache,
                                              void *v_cache, const int32_t *seqlens, int B, int H, int G, int d_h,
                                              int Tmax, float scale, int window, int split_tokens, gqa_dtype dtype,
                                              void *out, hipStream_t stream)
{
    char *ws = nullptr;
    if (B > 0) {
        gqa_status s = scratch_on_current_device(&ws);
        if (s != GQA_OK)
            return s;
    } else {
        // an empty batch queues nothing and needs no device address
        static char none;
        ws = &none;
    }
    return gqa::decode_step_in_workspace(q, k_new, v_new, k_cache, v_cache, seqlens, B, H, G, d_h, Tmax, scale,
                                         window, split_tokens, dtype, out, stream, ws, kScratchBytes);
}
