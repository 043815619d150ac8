// kernels.h -- launchers of the libgqa HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace gqa {

struct DecodeArgs {
    const void *q, *k, *v;          // k, v are written (position L_b) only when knew is set
    const void *knew, *vnew;        // appended token [B, G, D], or null
    const int32_t *seqlens;
    int B, H, G, D, Tmax;
    int window;                     // 0: every position
    float scale;
    void *out;
    float *part;  // partial rows (bf16 path)
    float *lse;   // partial base-2 log-sum-exp values (bf16 path)
    hipStream_t stream;
};

hipError_t launch_decode(const DecodePlan &plan, const DecodeArgs &args, gqa_dtype dtype);

// Workgroups of the plan's 16-bit decode variant (storage type, append or
// not) that fit on one compute unit.
hipError_t decode_blocks_per_cu(const DecodePlan &plan, int d_h, gqa_dtype dtype, bool append, int *blocks);

struct PrefillArgs {
    const void *q, *k, *v;
    int B, T, H, G, D;
    int causal;
    int window;  // causal sliding window (0: none): query t sees keys [t + 1 - window, t]
    void *out;
    hipStream_t stream;
};

hipError_t launch_prefill(const PrefillArgs &args, gqa_dtype dtype);

// weights: fp32 [H] per-head weights, or null for the plain mean.
hipError_t launch_mean_pool(const void *in, const float *weights, int64_t N, int H, int G, int D, gqa_dtype dtype,
                            void *out, hipStream_t stream);

// Debug builds: each kernel source file's range-check violation word (see
// GQA_IN_RANGE in device_common.h), read and cleared; 0 in release builds.
hipError_t debug_take_decode(unsigned int *w);
hipError_t debug_take_prefill(unsigned int *w);
hipError_t debug_take_pool(unsigned int *w);
// Debug builds: one range check that fails on purpose, guarding no memory
// access (pooling word, bit 7); hipErrorNotSupported in release builds.
hipError_t debug_selftest(hipStream_t stream);

}  // namespace gqa
