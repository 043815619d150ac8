// api_internal.h -- entry points shared between the C ABI translation units
// of libgqa (internal; not part of the public header).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "gqa.h"

namespace gqa {

// Records `msg` as the calling thread's last error text and returns `s`.
gqa_status set_last_error(gqa_status s, const std::string &msg);

// gqa_decode_step with the split workspace in caller-provided device memory
// of `ws_bytes` bytes: the library allocates nothing. A decode that needs
// more returns GQA_ERR_UNSUPPORTED before anything is queued.
gqa_status decode_step_in_workspace(const void *q, const void *k_new, const void *v_new, void *k_cache,
                                    void *v_cache, const int32_t *seqlens, int B, int H, int G, int d_h, int Tmax,
                                    float scale, int window, int split_tokens, gqa_dtype dtype, void *out,
                                    hipStream_t stream, char *ws, int64_t ws_bytes);

}  // namespace gqa
