// plan.h -- host-side argument checks and launch planning for libgqa.
// Pure C++: no HIP headers, so the same source builds into a host-only unit
// test with g++.
#pragma once

#include <cstdint>
#include <string>

#include "gqa.h"

namespace gqa {

// Decode launch plan. Heads of one key/value group are processed together in
// tiles of 16 * nt heads (the MFMA N dimension is 16); a group with more than
// 64 heads is covered by several head tiles.
struct DecodePlan {
    int r = 0;             // query heads per group, H / G
    int nt = 1;            // 16-head MFMA column tiles per workgroup: 1, 2 or 4
    int head_tiles = 1;    // ceil(r / (16 * nt))
    int chunk = 32;        // cache positions per workgroup (multiple of 32)
    int splits = 1;        // ceil(Tmax / chunk), at least 1
    int waves = 4;         // wavefronts per workgroup
    int64_t counter_offset = 0;  // byte offset of int32 arrival counters [B*G*head_tiles] (always 0)
    int64_t part_offset = 0;     // byte offset of fp32 partial outputs [B*H][splits][d_h]
    int64_t lse_offset = 0;      // byte offset of fp32 base-2 log-sum-exp [B*H][splits]
    int64_t n_counters = 0;
    int64_t workspace_bytes = 0; // 0 when splits == 1
};

constexpr int kDecodeTile = 32;      // cache positions per wavefront iteration
constexpr int kMinAutoChunk = 256;   // smallest automatic split

int64_t elem_size(gqa_dtype dt);
bool ranges_overlap(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes);

gqa_status check_decode(const void *q, const void *k, const void *v, const int32_t *seqlens, int B, int H,
                        int G, int d_h, int Tmax, float scale, gqa_dtype dtype, const void *out,
                        std::string *err);
gqa_status plan_decode(int B, int H, int G, int d_h, int Tmax, gqa_dtype dtype, int split_tokens,
                       int cu_count, DecodePlan *plan, std::string *err);
gqa_status check_prefill(const void *q, const void *k, const void *v, int B, int T, int H, int G, int d_h,
                         int causal, gqa_dtype dtype, const void *out, std::string *err);
gqa_status check_mean_pool(const void *in, int64_t N, int H, int G, int d_h, gqa_dtype dtype,
                           const void *out, std::string *err);

}  // namespace gqa
