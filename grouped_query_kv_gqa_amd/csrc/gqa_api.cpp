// gqa_api.cpp -- the C ABI of libgqa.so (declared in include/gqa.h).
//
// Every entry point checks its arguments on the host (plan.cpp) before it
// touches the HIP runtime, then queues its kernels on the caller's stream.
// The only state the library keeps is the split-decode workspace, one per
// (device, stream), grown on demand with stream-ordered allocation (policy in
// workspace.cpp), and cached device properties.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <string>
#include <unordered_map>

#include "gqa.h"
#include "kernels.h"
#include "api_internal.h"
#include "plan.h"
#include "workspace.h"

namespace {

thread_local std::string g_last_error;

gqa_status record(gqa_status s, const std::string &msg)
{
    g_last_error = msg;
    return s;
}

gqa_status hip_failure(hipError_t e, const char *where)
{
    g_last_error = std::string(where) + ": " + hipGetErrorString(e);
    return GQA_ERR_HIP;
}

// Device calls of the workspace registry, through the HIP runtime.
struct HipBackend final : gqa::WsBackend {
    int alloc(void **ptr, int64_t bytes, void *stream) override
    {
        return hipMallocAsync(ptr, static_cast<size_t>(bytes), static_cast<hipStream_t>(stream));
    }
    int free_async(void *ptr, void *stream) override
    {
        return hipFreeAsync(ptr, static_cast<hipStream_t>(stream));
    }
    int free_now(int device, void *ptr) override
    {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != device)
            e = hipSetDevice(device);
        if (e == hipSuccess)
            e = hipFreeAsync(ptr, nullptr);
        if (e == hipSuccess)
            e = hipStreamSynchronize(nullptr);
        if (cur != device)
            (void)hipSetDevice(cur);
        return e;
    }
    int sync_device(int device) override
    {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != device)
            e = hipSetDevice(device);
        if (e == hipSuccess)
            e = hipDeviceSynchronize();
        if (cur != device)
            (void)hipSetDevice(cur);
        return e;
    }
    int is_capturing(void *stream, bool *capturing) override
    {
        hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &st);
        *capturing = st != hipStreamCaptureStatusNone;
        return e;
    }
    std::string error_text(int code) override { return hipGetErrorString(static_cast<hipError_t>(code)); }
};

std::mutex g_mutex;
HipBackend g_backend;
gqa::WorkspaceRegistry g_workspaces(&g_backend);
std::unordered_map<int, int> g_cu_count;
std::unordered_map<int64_t, int> g_blocks_per_cu;  // variant key -> workgroups per CU

gqa_status cu_count(int device, int *out)
{
    auto it = g_cu_count.find(device);
    if (it != g_cu_count.end()) {
        *out = it->second;
        return GQA_OK;
    }
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess)
        return hip_failure(e, "hipDeviceGetAttribute");
    g_cu_count[device] = n;
    *out = n;
    return GQA_OK;
}

gqa_status blocks_per_cu(int device, const gqa::DecodePlan &p, int d_h, gqa_dtype dtype, bool append, int *out)
{
    const int64_t key =
        ((((((int64_t)device * 256 + d_h) * 8 + p.nt) * 16 + p.waves) * 16 + p.gb) * 4 + (int)dtype) * 2 + append;
    auto it = g_blocks_per_cu.find(key);
    if (it != g_blocks_per_cu.end()) {
        *out = it->second;
        return GQA_OK;
    }
    int n = 0;
    hipError_t e = gqa::decode_blocks_per_cu(p, d_h, dtype, append, &n);
    if (e != hipSuccess)
        return hip_failure(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    if (n < 1)
        n = 1;
    g_blocks_per_cu[key] = n;
    *out = n;
    return GQA_OK;
}

}  // namespace

namespace {

gqa_status decode_impl(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                       const void *v_cache, const int32_t *seqlens, int B, int H, int G, int d_h, int Tmax,
                       float scale, int window, int split_tokens, gqa_dtype dtype, void *out, hipStream_t stream,
                       char *fixed_ws, int64_t fixed_ws_bytes)
{
    std::string err;
    gqa_status s = gqa::check_decode_step(q, k_new, v_new, k_cache, v_cache, seqlens, B, H, G, d_h, Tmax, scale,
                                          window, dtype, out, &err);
    if (s != GQA_OK)
        return record(s, err);
    if (split_tokens < 0)
        return record(GQA_ERR_INVALID_ARG, "split_tokens must be >= 0");
    if (std::isnan(scale))
        scale = 1.0f / std::sqrt((float)d_h);
    gqa::DecodePlan plan;
    // sizes and launch limits, before anything touches the runtime
    if ((s = gqa::plan_decode(B, H, G, d_h, Tmax, dtype, split_tokens, 0, 0, &plan, &err)) != GQA_OK)
        return record(s, err);
    if (B == 0)
        return GQA_OK;

    std::lock_guard<std::mutex> lock(g_mutex);
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess)
        return hip_failure(e, "hipGetDevice");
    int cus = 0;
    if ((s = cu_count(device, &cus)) != GQA_OK)
        return s;
    const bool append = k_new != nullptr;
    gqa::DecodeArgs a{q, k_cache, v_cache, k_new, v_new, seqlens, B, H, G, d_h, Tmax, window, scale,
                      out, nullptr, nullptr, stream};
    if (dtype != GQA_FP32) {
        int bpc = 0;
        if ((s = blocks_per_cu(device, plan, d_h, dtype, append, &bpc)) != GQA_OK)
            return s;
        if ((s = gqa::plan_decode(B, H, G, d_h, Tmax, dtype, split_tokens, cus, bpc, &plan, &err)) != GQA_OK)
            return record(s, err);
        char *ws = nullptr;
        if (fixed_ws) {
            if (plan.workspace_bytes > fixed_ws_bytes)
                return record(GQA_ERR_UNSUPPORTED,
                              "this decode needs " + std::to_string(plan.workspace_bytes) +
                                  " bytes of scratch, above the fixed maximum of " + std::to_string(fixed_ws_bytes));
            ws = fixed_ws;
        } else {
            if ((s = g_workspaces.get(device, stream, plan.workspace_bytes, &ws, &err)) != GQA_OK)
                return record(s, err);
        }
        a.part = reinterpret_cast<float *>(ws + plan.part_offset);
        a.lse = reinterpret_cast<float *>(ws + plan.lse_offset);
    }
    e = gqa::launch_decode(plan, a, dtype);
    if (e != hipSuccess)
        return hip_failure(e, "decode launch");
    return GQA_OK;
}

}  // namespace

namespace gqa {

gqa_status set_last_error(gqa_status s, const std::string &msg)
{
    return record(s, msg);
}

gqa_status decode_step_in_workspace(const void *q, const void *k_new, const void *v_new, void *k_cache,
                                    void *v_cache, const int32_t *seqlens, int B, int H, int G, int d_h, int Tmax,
                                    float scale, int window, int split_tokens, gqa_dtype dtype, void *out,
                                    hipStream_t stream, char *ws, int64_t ws_bytes)
{
    if (!ws)
        return record(GQA_ERR_INVALID_ARG, "no workspace");
    return decode_impl(q, k_new, v_new, k_cache, v_cache, seqlens, B, H, G, d_h, Tmax, scale, window, split_tokens,
                       dtype, out, stream, static_cast<char *>(ws), ws_bytes);
}

}  // namespace gqa

extern "C" {

gqa_status gqa_decode_ex(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens, int B,
                         int H, int G, int d_h, int Tmax, float scale, gqa_dtype dtype, void *out,
                         hipStream_t stream, int split_tokens)
{
    return decode_impl(q, nullptr, nullptr, k_cache, v_cache, seqlens, B, H, G, d_h, Tmax, scale, 0, split_tokens,
                       dtype, out, stream, nullptr, 0);
}

gqa_status gqa_decode_step(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                           const int32_t *seqlens, int B, int H, int G, int d_h, int Tmax, float scale, int window,
                           int split_tokens, gqa_dtype dtype, void *out, hipStream_t stream)
{
    return decode_impl(q, k_new, v_new, k_cache, v_cache, seqlens, B, H, G, d_h, Tmax, scale, window, split_tokens,
                       dtype, out, stream, nullptr, 0);
}

gqa_status gqa_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens, int B,
                      int H, int G, int d_h, int Tmax, float scale, gqa_dtype dtype, void *out, hipStream_t stream)
{
    return gqa_decode_ex(q, k_cache, v_cache, seqlens, B, H, G, d_h, Tmax, scale, dtype, out, stream, 0);
}

gqa_status gqa_prefill_ex(const void *q, const void *k, const void *v, int B, int T, int H, int G, int d_h,
                          int causal, int window, gqa_dtype dtype, void *out, hipStream_t stream)
{
    std::string err;
    gqa_status s = gqa::check_prefill(q, k, v, B, T, H, G, d_h, causal, dtype, out, &err);
    if (s != GQA_OK)
        return record(s, err);
    if (window < 0)
        return record(GQA_ERR_INVALID_ARG, "window must be >= 0");
    if (window > 0 && !causal)
        return record(GQA_ERR_INVALID_ARG, "a sliding window needs causal = 1");
    if (B == 0 || T == 0)
        return GQA_OK;
    if ((s = gqa::check_prefill_launch(B, T, H, G, d_h, dtype, &err)) != GQA_OK)
        return record(s, err);
    gqa::PrefillArgs a{q, k, v, B, T, H, G, d_h, causal, window, out, stream};
    hipError_t e = gqa::launch_prefill(a, dtype);
    if (e != hipSuccess)
        return hip_failure(e, "prefill launch");
    return GQA_OK;
}

gqa_status gqa_prefill(const void *q, const void *k, const void *v, int B, int T, int H, int G, int d_h, int causal,
                       gqa_dtype dtype, void *out, hipStream_t stream)
{
    return gqa_prefill_ex(q, k, v, B, T, H, G, d_h, causal, 0, dtype, out, stream);
}

gqa_status gqa_mean_pool_kv(const void *in, int64_t N, int H, int G, int d_h, gqa_dtype dtype, void *out,
                            hipStream_t stream)
{
    std::string err;
    gqa_status s = gqa::check_mean_pool(in, N, H, G, d_h, dtype, out, &err);
    if (s != GQA_OK)
        return record(s, err);
    if (N == 0)
        return GQA_OK;
    hipError_t e = gqa::launch_mean_pool(in, nullptr, N, H, G, d_h, dtype, out, stream);
    if (e != hipSuccess)
        return hip_failure(e, "mean-pool launch");
    return GQA_OK;
}

gqa_status gqa_weighted_pool_kv(const void *in, const float *weights, int64_t N, int H, int G, int d_h,
                                gqa_dtype dtype, void *out, hipStream_t stream)
{
    std::string err;
    gqa_status s = gqa::check_mean_pool(in, N, H, G, d_h, dtype, out, &err);
    if (s != GQA_OK)
        return record(s, err);
    if (N == 0)
        return GQA_OK;
    if (!weights || (reinterpret_cast<uintptr_t>(weights) & 3u) != 0)
        return record(GQA_ERR_INVALID_ARG, "weights must be a non-null, 4-byte aligned fp32 array");
    if (gqa::ranges_overlap(out, N * G * d_h * gqa::elem_size(dtype), weights, 4 * (int64_t)H))
        return record(GQA_ERR_INVALID_ARG, "out overlaps weights");
    hipError_t e = gqa::launch_mean_pool(in, weights, N, H, G, d_h, dtype, out, stream);
    if (e != hipSuccess)
        return hip_failure(e, "weighted-pool launch");
    return GQA_OK;
}

gqa_status gqa_decode_plan(int B, int H, int G, int d_h, int Tmax, gqa_dtype dtype, int split_tokens, int cu_count,
                           int *chunk_tokens, int *num_splits, int64_t *workspace_bytes)
{
    std::string err;
    gqa::DecodePlan plan;
    gqa_status s = gqa::plan_decode(B, H, G, d_h, Tmax, dtype, split_tokens, cu_count, 0, &plan, &err);
    if (s != GQA_OK)
        return record(s, err);
    const bool fp32 = dtype == GQA_FP32 || B == 0;
    if (chunk_tokens)
        *chunk_tokens = fp32 ? Tmax : plan.full_P;
    if (num_splits)
        *num_splits = fp32 ? 1 : plan.nwg;
    if (workspace_bytes)
        *workspace_bytes = plan.workspace_bytes;
    return GQA_OK;
}

const char *gqa_status_string(gqa_status s)
{
    switch (s) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported";
    case GQA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *gqa_last_hip_error(void)
{
    return g_last_error.c_str();
}

const char *gqa_last_error(void)
{
    return g_last_error.c_str();
}

gqa_status gqa_release_workspaces(void)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    std::string err;
    gqa_status s = g_workspaces.release_all(&err);
    if (s != GQA_OK)
        return record(s, err);
    return GQA_OK;
}

int gqa_abi_version(void)
{
    return 2;
}

gqa_status gqa_debug_checks(int *enabled, uint32_t *flags)
{
#ifdef GQA_DEBUG
    constexpr int on = 1;
#else
    constexpr int on = 0;
#endif
    if (enabled)
        *enabled = on;
    uint32_t f = 0;
    if (on) {
        hipError_t e = hipDeviceSynchronize();
        unsigned int w = 0;
        if (e == hipSuccess && (e = gqa::debug_take_decode(&w)) == hipSuccess)
            f |= w & 0xffffu;
        if (e == hipSuccess && (e = gqa::debug_take_prefill(&w)) == hipSuccess)
            f |= (w & 0xffu) << 16;
        if (e == hipSuccess && (e = gqa::debug_take_pool(&w)) == hipSuccess)
            f |= (w & 0xffu) << 24;
        if (e != hipSuccess)
            return hip_failure(e, "debug check words");
    }
    if (flags)
        *flags = f;
    return GQA_OK;
}

gqa_status gqa_debug_selftest(hipStream_t stream)
{
    const hipError_t e = gqa::debug_selftest(stream);
    if (e == hipErrorNotSupported)
        return record(GQA_ERR_UNSUPPORTED, "range checks are compiled only into libgqa_debug.so");
    if (e != hipSuccess)
        return hip_failure(e, "debug self-test launch");
    return GQA_OK;
}

}  // extern "C"
