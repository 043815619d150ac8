// plan.h -- host-side argument checks and launch planning for libgqa.
// Pure C++: no HIP headers, so the same source builds into a host-only unit
// test with g++.
#pragma once

#include <cstdint>
#include <string>

#include "gqa.h"

namespace gqa {

// Decode launch plan. The cache positions of all sequences, laid end to end,
// are cut into equal pieces, one per workgroup along grid x; grid y covers
// (group blocks of gb key/value groups) x (head tiles of 16*nt query heads),
// or the G groups for the wide kernel.
struct DecodePlan {
    int r = 0;           // query heads per group, H / G
    int wide = 0;        // 1: groups of 33..64 heads, one 8-wave workgroup per (slice, group) with LDS stages
    int nt = 1;          // 16-head MFMA column tiles per wave: 1 or 2
    int head_tiles = 1;  // ceil(r / (16 * nt))
    int waves = 8;       // wavefronts per workgroup
    int gb = 1;          // key/value groups per workgroup; waves / gb waves share a group
    int nwg = 1;         // workgroups along the flat position space (grid x)
    int fixed_P = 0;     // piece length when set by the caller, else 0 (balanced on the device)
    int full_P = 32;     // piece length when every sequence has Tmax positions
    int startup = 0;     // virtual positions before each sequence (the cost of starting a piece); 0 with
                         // fixed_P; negative: that many, where the kernels find it leaves P unchanged
    int merge_nq = 8;    // merge kernel: d-quads per wave (64/merge_nq lanes share a quad)
    int merge_u = 4;     // merge kernel: pieces each slot lane loads per round (4 or 16)
    int64_t part_offset = 0;      // fp32 partial rows [nwg + B][H][d_h]
    int64_t lse_offset = 0;       // fp32 base-2 log-sum-exp [nwg + B][H]
    int64_t workspace_bytes = 0;  // 0 for the fp32 path
};

constexpr int kDecodeTile = 32;  // cache positions per wavefront iteration
// Bytes a workgroup could have streamed in the time it spends starting a
// piece (the first stages' round trip, then the combine and stores at its
// end), about 5-10 us at a compute unit's share of the bandwidth: the
// balanced partition of the wide kernel charges each sequence this many
// bytes' worth of positions (measured on the multi-query batch: none
// 40.0 us, 64 KiB 39.2 us, 128 KiB 38.8 us, 256 KiB 38.2 us; on another GPU
// 256 KiB 39.1-39.3 us, 384 KiB 38.9 us, 512 KiB 38.8-38.9 us, 768 KiB
// 39.6-39.7 us, 1 MiB 40.0-40.2 us).
constexpr int64_t kPieceStartupBytes = 512 * 1024;

// Workgroups of a decode variant that fit on one compute unit, as measured
// for the gfx950 build (used when the runtime is not asked).
int default_blocks_per_cu(int d_h, int nt);

int64_t elem_size(gqa_dtype dt);
bool ranges_overlap(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes);

gqa_status check_decode(const void *q, const void *k, const void *v, const int32_t *seqlens, int B, int H,
                        int G, int d_h, int Tmax, float scale, gqa_dtype dtype, const void *out,
                        std::string *err);
gqa_status plan_decode(int B, int H, int G, int d_h, int Tmax, gqa_dtype dtype, int split_tokens,
                       int cu_count, int blocks_per_cu, DecodePlan *plan, std::string *err);
// check_decode plus the cache-append and window arguments of gqa_decode_step.
gqa_status check_decode_step(const void *q, const void *k_new, const void *v_new, const void *k, const void *v,
                             const int32_t *seqlens, int B, int H, int G, int d_h, int Tmax, float scale, int window,
                             gqa_dtype dtype, const void *out, std::string *err);

gqa_status check_prefill(const void *q, const void *k, const void *v, int B, int T, int H, int G, int d_h,
                         int causal, gqa_dtype dtype, const void *out, std::string *err);
// Grid and index limits of the prefill launch (after check_prefill).
constexpr int kPrefillRows = 256;  // query rows (token x head) per MFMA prefill workgroup
gqa_status check_prefill_launch(int B, int T, int H, int G, int d_h, gqa_dtype dtype, std::string *err);
gqa_status check_mean_pool(const void *in, int64_t N, int H, int G, int d_h, gqa_dtype dtype,
                           const void *out, std::string *err);

}  // namespace gqa
