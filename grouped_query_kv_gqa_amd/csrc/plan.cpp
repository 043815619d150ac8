// plan.cpp -- host-side argument checks and launch planning for libgqa.
// Pure C++ (no HIP); see plan.h.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>

namespace gqa {

namespace {

gqa_status fail(std::string *err, gqa_status s, const std::string &msg)
{
    if (err)
        *err = msg;
    return s;
}

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int64_t ceil_div(int64_t a, int64_t b)
{
    return (a + b - 1) / b;
}

int64_t round_up(int64_t a, int64_t m)
{
    return ceil_div(a, m) * m;
}

bool dtype_ok(gqa_dtype dt)
{
    return dt == GQA_BF16 || dt == GQA_FP32 || dt == GQA_FP16;
}

}  // namespace

int64_t elem_size(gqa_dtype dt)
{
    return dt == GQA_FP32 ? 4 : 2;
}

bool ranges_overlap(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes)
{
    if (!a || !b || a_bytes <= 0 || b_bytes <= 0)
        return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(b_bytes) && b0 < a0 + static_cast<uintptr_t>(a_bytes);
}

gqa_status check_decode(const void *q, const void *k, const void *v, const int32_t *seqlens, int B, int H,
                        int G, int d_h, int Tmax, float scale, gqa_dtype dtype, const void *out,
                        std::string *err)
{
    if (B < 0 || Tmax < 0)
        return fail(err, GQA_ERR_INVALID_ARG, "B and Tmax must be >= 0");
    if (H < 1 || G < 1 || d_h < 1)
        return fail(err, GQA_ERR_INVALID_ARG, "H, G and d_h must be >= 1");
    if (H % G != 0)
        return fail(err, GQA_ERR_INVALID_ARG, "G must divide H");
    if (!dtype_ok(dtype))
        return fail(err, GQA_ERR_UNSUPPORTED, "unknown dtype");
    if (d_h != 64 && d_h != 128)
        return fail(err, GQA_ERR_UNSUPPORTED, "d_h must be 64 or 128");
    if (std::isinf(scale))  // NaN selects 1/sqrt(d_h)
        return fail(err, GQA_ERR_INVALID_ARG, "scale must be finite (or NaN for 1/sqrt(d_h))");
    if (B == 0)
        return GQA_OK;
    if (!q || !seqlens || !out || (Tmax > 0 && (!k || !v)))
        return fail(err, GQA_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(q) || !aligned16(out) || (Tmax > 0 && (!aligned16(k) || !aligned16(v))))
        return fail(err, GQA_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
    const int64_t e = elem_size(dtype);
    const int64_t q_bytes = (int64_t)B * H * d_h * e;
    const int64_t kv_bytes = (int64_t)B * Tmax * G * d_h * e;
    if (ranges_overlap(out, q_bytes, q, q_bytes) || ranges_overlap(out, q_bytes, k, kv_bytes) ||
        ranges_overlap(out, q_bytes, v, kv_bytes) || ranges_overlap(out, q_bytes, seqlens, 4 * (int64_t)B))
        return fail(err, GQA_ERR_INVALID_ARG, "out overlaps an input");
    return GQA_OK;
}

gqa_status check_decode_step(const void *q, const void *k_new, const void *v_new, const void *k, const void *v,
                             const int32_t *seqlens, int B, int H, int G, int d_h, int Tmax, float scale, int window,
                             gqa_dtype dtype, const void *out, std::string *err)
{
    gqa_status s = check_decode(q, k, v, seqlens, B, H, G, d_h, Tmax, scale, dtype, out, err);
    if (s != GQA_OK)
        return s;
    if (window < 0)
        return fail(err, GQA_ERR_INVALID_ARG, "window must be >= 0");
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(err, GQA_ERR_INVALID_ARG, "k_new and v_new must both be given or both be null");
    if (B == 0 || !k_new)
        return GQA_OK;
    if (Tmax < 1)
        return fail(err, GQA_ERR_INVALID_ARG, "appending needs Tmax >= 1");
    if (!aligned16(k_new) || !aligned16(v_new))
        return fail(err, GQA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
    const int64_t e = elem_size(dtype);
    const int64_t q_bytes = (int64_t)B * H * d_h * e;
    const int64_t n_bytes = (int64_t)B * G * d_h * e;
    const int64_t kv_bytes = (int64_t)B * Tmax * G * d_h * e;
    if (ranges_overlap(out, q_bytes, k_new, n_bytes) || ranges_overlap(out, q_bytes, v_new, n_bytes))
        return fail(err, GQA_ERR_INVALID_ARG, "out overlaps an input");
    // the caches are written: they must not overlap each other or any input
    const void *ins[] = {q, k_new, v_new, seqlens};
    const int64_t in_bytes[] = {q_bytes, n_bytes, n_bytes, 4 * (int64_t)B};
    if (ranges_overlap(k, kv_bytes, v, kv_bytes))
        return fail(err, GQA_ERR_INVALID_ARG, "k_cache and v_cache overlap");
    for (int i = 0; i < 4; ++i)
        if (ranges_overlap(k, kv_bytes, ins[i], in_bytes[i]) || ranges_overlap(v, kv_bytes, ins[i], in_bytes[i]))
            return fail(err, GQA_ERR_INVALID_ARG, "a cache overlaps q, k_new, v_new or seqlens");
    return GQA_OK;
}

int default_blocks_per_cu(int d_h, int nt)
{
    // gfx950 build: d_h = 64 with 32-head tiles runs two 4-wave workgroups per
    // CU; every other variant is register-limited to one workgroup per CU.
    return (d_h == 64 && nt == 2) ? 2 : 1;
}

gqa_status plan_decode(int B, int H, int G, int d_h, int Tmax, gqa_dtype dtype, int split_tokens,
                       int cu_count, int blocks_per_cu, DecodePlan *plan, std::string *err)
{
    if (B < 0 || Tmax < 0 || H < 1 || G < 1 || d_h < 1)
        return fail(err, GQA_ERR_INVALID_ARG, "bad sizes");
    if (H % G != 0)
        return fail(err, GQA_ERR_INVALID_ARG, "G must divide H");
    if (!dtype_ok(dtype))
        return fail(err, GQA_ERR_UNSUPPORTED, "unknown dtype");
    if (d_h != 64 && d_h != 128)
        return fail(err, GQA_ERR_UNSUPPORTED, "d_h must be 64 or 128");
    if (split_tokens < 0)
        return fail(err, GQA_ERR_INVALID_ARG, "split_tokens must be >= 0");
    DecodePlan p;
    p.r = H / G;
    if (p.r > 32 && p.r <= 64) {
        // Wide groups: one 8-wave workgroup per (slice, group) stages the
        // group's rows in LDS once for all its heads (2 tiles of 32 heads x
        // 4 position phases).
        p.wide = 1;
        p.nt = 2;
        p.head_tiles = 1;
        p.waves = 8;
        p.gb = 1;
    } else {
        // Groups wider than 16 heads take 32-head tiles (more head tiles run
        // as more workgroups over the same positions). One 16-head tile per
        // wave leaves room for 8-wave workgroups; wider tiles need the
        // registers of 4-wave workgroups.
        p.nt = p.r <= 16 ? 1 : 2;
        p.head_tiles = (int)ceil_div(p.r, 16 * p.nt);
        p.waves = p.nt == 1 ? 8 : 4;
        p.gb = 1;
        for (int c : {8, 4, 2}) {
            if (c <= p.waves && G % c == 0) {
                p.gb = c;
                break;
            }
        }
    }
    // Launch limits, checked here so that gqa_decode_plan and gqa_decode
    // agree: the merge grid has one row of workgroups per sequence (at most
    // 65535), flat positions are 32-bit on the device, and a launch holds
    // fewer than 2^32 work-items along x.
    if (B > 65535)
        return fail(err, GQA_ERR_UNSUPPORTED, "B must be <= 65535");
    if ((int64_t)B * Tmax > 0x7fffffff)
        return fail(err, GQA_ERR_UNSUPPORTED, "B * Tmax must be below 2^31");
    if (dtype == GQA_FP32 || B == 0) {
        if ((int64_t)B * H * 64 > 0xffffffffLL)
            return fail(err, GQA_ERR_UNSUPPORTED, "B * H must be below 2^26 on the fp32 path");
        p.nwg = 0;
        if (plan)
            *plan = p;
        return GQA_OK;
    }
    const int64_t combos = (int64_t)(G / p.gb) * p.head_tiles;
    if (combos > 65535)
        return fail(err, GQA_ERR_UNSUPPORTED, "too many key/value heads");
    // Startup positions for the wide kernel: the piece startup cost over the
    // bytes a workgroup streams per position (one group's K and V rows). The
    // narrow kernel reads 8 groups per position, where a piece's start costs
    // about one tile; a fixed charge there measured slower, since in uniform
    // batches it moves slice boundaries off sequence boundaries (giving
    // workgroups two pieces each) and can raise the tile-rounded slice
    // length, so the narrow kernel's charge below is conditional.
    if (split_tokens == 0 && p.wide) {
        const int64_t per_pos = (int64_t)p.gb * d_h * 2 * elem_size(dtype);
        p.startup = (int)std::min<int64_t>(kPieceStartupBytes / per_pos, 4096);
        if ((int64_t)B * (Tmax + p.startup) > 0x7fffffff)
            p.startup = 0;  // keep flat positions within 31 bits
    }
    // Narrow kernel: a one-tile charge per sequence, which the kernels apply
    // only when it leaves the tile-rounded slice length unchanged (negative:
    // decided on the device from the lengths).
    if (split_tokens == 0 && !p.wide && (int64_t)B * (Tmax + kDecodeTile) <= 0x7fffffff)
        p.startup = -kDecodeTile;
    const int64_t positions = (int64_t)B * (Tmax + std::max(p.startup, 0));
    const int64_t max_pieces = ceil_div(positions > 0 ? positions : 1, kDecodeTile);
    int64_t nwg;
    if (split_tokens > 0) {
        p.fixed_P = (int)round_up(split_tokens, kDecodeTile);
        nwg = ceil_div(positions > 0 ? positions : 1, p.fixed_P);
        p.full_P = p.fixed_P;
    } else {
        const int64_t cus = cu_count > 0 ? cu_count : 256;
        const int64_t bpc = blocks_per_cu > 0 ? blocks_per_cu : (p.wide ? 1 : default_blocks_per_cu(d_h, p.nt));
        nwg = (cus * bpc) / combos;
        if (nwg < 1)
            nwg = 1;
        if (nwg > max_pieces)
            nwg = max_pieces;
        int64_t P = round_up(ceil_div(positions > 0 ? positions : 1, nwg), kDecodeTile);
        p.full_P = (int)(P < kDecodeTile ? kDecodeTile : P);
    }
    if (nwg * p.waves * 64 > 0xffffffffLL)
        return fail(err, GQA_ERR_UNSUPPORTED, "too many cache positions for the split size");
    p.nwg = (int)nwg;
    // Merge layout: enough slot lanes that each takes at most U pieces of a
    // full-length row, the rest of the 64 lanes spread over d. U = 4, or 16
    // when a row can hold more than 128 pieces (measured on the 131072-token
    // sequence, 257 pieces: 91.6-91.8 us against 93.0-93.2 us with U = 4;
    // on the Llama-3-8B layer, 17 pieces, U = 16 was 0.6 us slower).
    {
        const int64_t exp_slots = ceil_div(Tmax > 0 ? Tmax : 1, p.full_P) + 1;
        const int u = exp_slots > 128 ? 16 : 4;
        int64_t ns = 1;
        while (ns < 64 && ns * u < exp_slots)
            ns *= 2;
        const int64_t min_ns = 256 / d_h;  // at most d_h / 4 quads
        if (ns < min_ns)
            ns = min_ns;
        p.merge_nq = (int)(64 / ns);
        p.merge_u = u;
    }
    // One partial row per (piece, head): the waves that share a group combine
    // their states inside the workgroup before anything is written.
    const int64_t slots = (nwg + B) * (int64_t)H;
    p.part_offset = 0;
    p.lse_offset = round_up(slots * d_h * 4, 256);
    p.workspace_bytes = round_up(p.lse_offset + slots * 4, 256);
    if (plan)
        *plan = p;
    return GQA_OK;
}

gqa_status check_prefill(const void *q, const void *k, const void *v, int B, int T, int H, int G, int d_h,
                         int causal, gqa_dtype dtype, const void *out, std::string *err)
{
    if (B < 0 || T < 0)
        return fail(err, GQA_ERR_INVALID_ARG, "B and T must be >= 0");
    if (H < 1 || G < 1 || d_h < 1)
        return fail(err, GQA_ERR_INVALID_ARG, "H, G and d_h must be >= 1");
    if (H % G != 0)
        return fail(err, GQA_ERR_INVALID_ARG, "G must divide H");
    if (causal != 0 && causal != 1)
        return fail(err, GQA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!dtype_ok(dtype))
        return fail(err, GQA_ERR_UNSUPPORTED, "unknown dtype");
    if (d_h != 64 && d_h != 128)
        return fail(err, GQA_ERR_UNSUPPORTED, "d_h must be 64 or 128");
    if (B == 0 || T == 0)
        return GQA_OK;
    if (!q || !k || !v || !out)
        return fail(err, GQA_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(err, GQA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    const int64_t e = elem_size(dtype);
    const int64_t q_bytes = (int64_t)B * T * H * d_h * e;
    const int64_t kv_bytes = (int64_t)B * T * G * d_h * e;
    if (ranges_overlap(out, q_bytes, q, q_bytes) || ranges_overlap(out, q_bytes, k, kv_bytes) ||
        ranges_overlap(out, q_bytes, v, kv_bytes))
        return fail(err, GQA_ERR_INVALID_ARG, "out overlaps an input");
    return GQA_OK;
}

gqa_status check_prefill_launch(int B, int T, int H, int G, int d_h, gqa_dtype dtype, std::string *err)
{
    // grid y = G and z = B (each at most 65535); fewer than 2^32 work-items
    // along x; 31-bit row indices inside the kernels.
    if (B > 65535 || G > 65535)
        return fail(err, GQA_ERR_UNSUPPORTED, "B and G must be <= 65535");
    const int64_t rows = (int64_t)B * T * H;
    if (rows > 0x7fffffff)
        return fail(err, GQA_ERR_UNSUPPORTED, "B * T * H must be below 2^31");
    const int r = H / G;
    const bool row_kernel = dtype == GQA_FP32 || r > kPrefillRows;
    if (row_kernel && rows * 64 > 0xffffffffLL)
        return fail(err, GQA_ERR_UNSUPPORTED, "B * T * H must be below 2^26 on the row-per-wave path");
    (void)d_h;
    return GQA_OK;
}

gqa_status check_mean_pool(const void *in, int64_t N, int H, int G, int d_h, gqa_dtype dtype,
                           const void *out, std::string *err)
{
    if (N < 0)
        return fail(err, GQA_ERR_INVALID_ARG, "N must be >= 0");
    if (H < 1 || G < 1 || d_h < 1)
        return fail(err, GQA_ERR_INVALID_ARG, "H, G and d_h must be >= 1");
    if (H % G != 0)
        return fail(err, GQA_ERR_INVALID_ARG, "G must divide H");
    if (!dtype_ok(dtype))
        return fail(err, GQA_ERR_UNSUPPORTED, "unknown dtype");
    if (d_h % 8 != 0)
        return fail(err, GQA_ERR_UNSUPPORTED, "d_h must be a multiple of 8");
    if (N == 0)
        return GQA_OK;
    if (!in || !out)
        return fail(err, GQA_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(in) || !aligned16(out))
        return fail(err, GQA_ERR_INVALID_ARG, "in and out must be 16-byte aligned");
    const int64_t e = elem_size(dtype);
    if (ranges_overlap(out, N * G * d_h * e, in, N * H * d_h * e))
        return fail(err, GQA_ERR_INVALID_ARG, "out overlaps in");
    return GQA_OK;
}

}  // namespace gqa
