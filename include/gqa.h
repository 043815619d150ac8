/*
 * gqa.h -- C ABI of libgqa.so: grouped-query attention (GQA) forward over a
 * key/value cache on AMD Instinct MI355X (gfx950).
 *
 * The operation (sources are web pages; each call below names its passage):
 *   H query heads are split into G contiguous groups of r = H/G heads; query
 *   head h (0-indexed) reads key/value head g(h) = floor(h*G/H) = h / r, which
 *   is the 1-indexed rule g(i) = ceil(i*G/H) of "Grouped-Query Attention"
 *   (llm-arch-kb), section 2 Derivation, The grouping. Each head then does
 *   ordinary scaled dot-product attention against its group's keys and values
 *   (same page, section 3 Reference implementation: scores divided by
 *   sqrt(d_h), causal mask, softmax over keys, times v). G = H is multi-head
 *   attention and G = 1 is multi-query attention (same page, section 1
 *   Premise; crackai.dev paper card, How It Works).
 *
 * Conventions shared by every call:
 *   - Tensors are dense, row-major, caller-owned DEVICE memory with the head
 *     dimension d_h innermost and contiguous. The library keeps no pointer
 *     after a call returns and never frees caller memory.
 *   - One dtype for all floating-point tensors of a call: GQA_BF16 (bf16
 *     storage, fp32 accumulation and softmax, bf16 output rounded to nearest
 *     even), GQA_FP16 (the same with IEEE fp16 storage and fp16 MFMA inputs;
 *     the pages' own cache arithmetic counts 2-byte fp16 scalars: "Grouped-Query
 *     Attention" (llm-arch-kb), section 2 Derivation, KV-cache footprint) or
 *     GQA_FP32 (fp32 storage, outputs and softmax sums; a debug path whose
 *     scores and running maxima are kept in fp64, so that its probabilities
 *     keep fp32 accuracy when scores are large).
 *   - Calls are asynchronous on `stream` (0 = the null stream): they return
 *     once the work is queued. Work on one stream runs in order.
 *   - All argument checks run on the host before anything is queued. A
 *     failing check returns a status and queues nothing. `out` must not
 *     overlap any input. q, k, v and out must be 16-byte aligned.
 *   - A batch of zero sequences (B = 0, or N = 0 for pooling) is valid and
 *     queues nothing; its pointers may be NULL.
 *   - GQA_ERR_HIP means the HIP runtime reported an error while queueing;
 *     gqa_last_hip_error() then holds its text.
 *   - Thread safety: calls may be made from several host threads. Calls that
 *     share a stream are serialised by that stream.
 */
#ifndef GQA_H_
#define GQA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t; /* same type as HIP's own typedef */

typedef enum gqa_status {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = 1, /* null pointer, negative size, G not dividing H, misalignment, aliasing */
    GQA_ERR_UNSUPPORTED = 2, /* valid but not built: d_h other than 64 or 128, unknown dtype */
    GQA_ERR_HIP = 3          /* the HIP runtime failed; see gqa_last_hip_error() */
} gqa_status;

typedef enum gqa_dtype { GQA_BF16 = 0, GQA_FP32 = 1, GQA_FP16 = 2 } gqa_dtype;

/*
 * gqa_decode -- one decode step: one new query per sequence against that
 * sequence's whole cache.
 * Defines: "Grouped-Query Attention" (llm-arch-kb), section 1 Premise (at a
 * decode step every cached key and value is read to produce one token) and
 * section 2 Derivation (head i attends over its cached keys and values; The
 * grouping assigns head i to group g(i)).
 *
 *   q        [B, H, d_h]        the new queries
 *   k_cache  [B, Tmax, G, d_h]  keys; position t of sequence b is k_cache[b, t]
 *   v_cache  [B, Tmax, G, d_h]  values, same layout
 *   seqlens  [B] int32, DEVICE memory: sequence b attends over positions
 *            [0, L_b) with L_b = min(max(seqlens[b], 0), Tmax). Positions at or
 *            beyond L_b are never read and may hold anything (NaN included).
 *            L_b = 0 gives an all-zero output row. Whether the newest token's
 *            key and value are among the L_b positions is the caller's choice.
 *   scale    multiplies q.k before the softmax (1/sqrt(d_h) for the pages'
 *            attention); finite, or NaN to select 1/sqrt(d_h).
 *   out      [B, H, d_h]        same dtype as q
 *   out[b,h,:] = sum_t softmax_t(scale * q[b,h,:].k_cache[b,t,g(h),:]) v_cache[b,t,g(h),:]
 *
 * Work is balanced over the GPU by laying all sequences' cache positions
 * end to end and giving every workgroup an equal slice; a sequence cut over
 * several slices is merged with a log-sum-exp combine in a second launch on
 * the same stream. Results are bit-identical from call to call.
 *
 * Workspace. The fp32 partial rows live in a library-owned block of device
 * memory, one per (device, stream): allocated with stream-ordered allocation
 * (hipMallocAsync on `stream`) by the first 16-bit call that needs it and
 * replaced by a larger one when a later call needs more. Calls on one stream
 * are ordered by that stream; calls on different streams use different
 * blocks. gqa_release_workspaces() frees them all. Blocks are keyed by the
 * stream handle: a destroyed stream's block stays allocated, and a stream
 * created later with the same handle takes it over, so call
 * gqa_release_workspaces() after destroying streams whose work may still be
 * running.
 *
 * Graph capture. A call made while `stream` is being captured never
 * allocates: if the stream's workspace is missing or too small it returns
 * GQA_ERR_INVALID_ARG and queues nothing, so make one eager call of the same
 * (or a larger) shape on the capture stream first. The captured graph keeps
 * the block's address and reads seqlens and the tensors at replay time. A
 * block that a captured graph references is never freed when a later, larger
 * eager call replaces it (it is kept until gqa_release_workspaces), so the
 * graph stays valid. The graph shares the block with every other call on
 * its capture stream: replaying it while such a call (or another graph
 * captured on that stream) runs on a different stream races. Callers that
 * cannot allocate at all use gqa_decode_step_noalloc instead.
 * Requires 1 <= G, G divides H, Tmax >= 0, d_h in {64, 128}; B <= 65535 and
 * B * Tmax < 2^31 (else GQA_ERR_UNSUPPORTED).
 */
gqa_status gqa_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens,
                      int B, int H, int G, int d_h, int Tmax, float scale, gqa_dtype dtype, void *out,
                      hipStream_t stream);

/*
 * gqa_decode_ex -- gqa_decode with an explicit slice length: every
 * workgroup takes `split_tokens` consecutive positions (rounded up to a
 * multiple of 32) of the end-to-end position space, instead of an equal share
 * of it. 0 selects the equal share gqa_decode uses. Results agree with
 * gqa_decode up to fp32 rounding of the combine. The fp32 path ignores
 * split_tokens. Same source passages as gqa_decode.
 */
gqa_status gqa_decode_ex(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens,
                         int B, int H, int G, int d_h, int Tmax, float scale, gqa_dtype dtype, void *out,
                         hipStream_t stream, int split_tokens);

/*
 * gqa_decode_step -- one decode step of a serving loop, with two optional
 * variants: the new token's key and value are appended to the cache before
 * it is read, and each query may see only a sliding window of the newest
 * positions.
 * Defines: "Grouped-Query Attention" (llm-arch-kb), section 1 Premise (a
 * decode step reads every cached entry, the new token's included) and section
 * 2 Derivation, Setup (head i attends over the keys and values cached so
 * far); section 4 Empirical evidence, Mistral 7B ablation (GQA combined with
 * sliding-window attention; the page gives no formula, the window below is
 * this library's reading).
 *
 *   k_new, v_new  [B, G, d_h] the new token's key and value, or both NULL
 *                 (no append). With them, for each b with L0 = clamp(seqlens[b],
 *                 0, Tmax) < Tmax, k_new[b] and v_new[b] are written to cache
 *                 position L0 and the sequence is attended over L0 + 1
 *                 positions; a full cache (L0 = Tmax) is neither written nor
 *                 extended. seqlens itself is not modified (the caller
 *                 advances it).
 *   k_cache, v_cache  as for gqa_decode, written at position L0 when
 *                 appending; they must not overlap each other or any input.
 *   window        0: every position; W > 0: only the W newest positions
 *                 [max(0, L - W), L) of the (appended) sequence are read.
 *   split_tokens  as for gqa_decode_ex.
 * Other arguments, layouts and errors as for gqa_decode; window < 0 and one
 * of k_new, v_new NULL without the other are GQA_ERR_INVALID_ARG.
 */
gqa_status gqa_decode_step(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                           const int32_t *seqlens, int B, int H, int G, int d_h, int Tmax, float scale, int window,
                           int split_tokens, gqa_dtype dtype, void *out, hipStream_t stream);

/*
 * gqa_decode_step_noalloc -- gqa_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, kernels and results as
 * gqa_decode_step (bit for bit), but the split workspace is a fixed 32 MiB
 * device array inside the library, one per GPU, held until the process ends:
 * nothing is allocated or freed. A decode whose workspace would exceed it
 * ((splits + B) * H * (d_h + 1) * 4 bytes, with the split count from
 * gqa_decode_plan; about 10 MB for 64 sequences of 64 heads at d_h = 128)
 * returns GQA_ERR_UNSUPPORTED and queues nothing. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or concurrent graph replays) race and must be
 * serialised by the caller. The array needs no clearing between calls.
 */
gqa_status gqa_decode_step_noalloc(const void *q, const void *k_new, const void *v_new, void *k_cache,
                                   void *v_cache, const int32_t *seqlens, int B, int H, int G, int d_h, int Tmax,
                                   float scale, int window, int split_tokens, gqa_dtype dtype, void *out,
                                   hipStream_t stream);

/*
 * gqa_prefill -- attention for every position of B sequences of length T.
 * Defines: "Grouped-Query Attention" (llm-arch-kb), section 3 Reference
 * implementation (sketch: q [B,T,H,d_h], k and v [B,T,G,d_h] broadcast to the
 * H query heads group by group, scores divided by sqrt(d_h), causal mask,
 * softmax over keys, times v).
 *
 *   q       [B, T, H, d_h]
 *   k, v    [B, T, G, d_h]
 *   causal  1: query position t attends to key positions s <= t (diagonal
 *           kept); 0: to every position.
 *   out     [B, T, H, d_h]   attention output before the output projection
 *   The scale is fixed at 1/sqrt(d_h).
 * Requires G divides H, T >= 0, d_h in {64, 128}.
 */
gqa_status gqa_prefill(const void *q, const void *k, const void *v, int B, int T, int H, int G, int d_h,
                       int causal, gqa_dtype dtype, void *out, hipStream_t stream);

/*
 * gqa_prefill_ex -- gqa_prefill with a causal sliding window: query position
 * t attends to key positions [max(0, t + 1 - window), t], the `window` newest
 * ones with itself included. window = 0 is gqa_prefill.
 * Defines: "Grouped-Query Attention" (llm-arch-kb), section 3 Reference
 * implementation (the causal attention above) and section 4 Empirical
 * evidence, Mistral 7B ablation (GQA paired with sliding-window attention;
 * the window bounds above are this library's reading, the page gives none).
 * window < 0, or window > 0 with causal = 0, is GQA_ERR_INVALID_ARG. Other
 * arguments as for gqa_prefill.
 */
gqa_status gqa_prefill_ex(const void *q, const void *k, const void *v, int B, int T, int H, int G, int d_h,
                          int causal, int window, gqa_dtype dtype, void *out, hipStream_t stream);

/*
 * gqa_mean_pool_kv -- convert multi-head key or value heads into G groups by
 * averaging the r = H/G heads of each group.
 * Defines: "Grouped-Query Attention" (llm-arch-kb), section 2 Derivation,
 * Uptraining recipe (each group starts as the mean of the original heads
 * assigned to it); crackai.dev paper card, How It Works (mean-pool the
 * key/value heads within each group).
 *
 *   in   [N, H, d_h]  a weight matrix [d, H*d_h] viewed with N = d, or
 *                     projected keys/values [tokens, H*d_h] with N = tokens
 *   out  [N, G, d_h]  out[n,g,:] = (1/r) * sum_{j<r} in[n, g*r + j, :],
 *                     accumulated in fp32; G = H copies exactly
 * Requires G divides H, N >= 0, d_h >= 1 with d_h a multiple of 8.
 */
gqa_status gqa_mean_pool_kv(const void *in, int64_t N, int H, int G, int d_h, gqa_dtype dtype, void *out,
                            hipStream_t stream);

/*
 * gqa_decode_plan -- the bf16 decode partition gqa_decode_ex would use,
 * computed on the host without touching the GPU (assuming the occupancy of
 * the gfx950 build; the library itself asks the runtime): `num_splits`
 * workgroups along the end-to-end position space, `chunk_tokens` positions
 * per workgroup when every sequence holds Tmax positions (shorter sequences
 * shrink the slice on the device), and the workspace bytes. For groups of
 * 33 to 64 heads with split_tokens = 0, each sequence is also charged
 * startup positions (512 KiB divided by the K/V bytes a workgroup reads per
 * position), the cost of starting a piece, so that workgroups holding the
 * start of a sequence take fewer real positions. For the fp32
 * path: chunk_tokens = Tmax, num_splits = 1, workspace 0. `cu_count` is the
 * GPU's compute-unit count (256 on MI355X). Any output pointer may be NULL.
 * Returns GQA_OK or the status gqa_decode would return for the same sizes
 * (the size and launch-limit checks are shared).
 */
gqa_status gqa_decode_plan(int B, int H, int G, int d_h, int Tmax, gqa_dtype dtype, int split_tokens,
                           int cu_count, int *chunk_tokens, int *num_splits, int64_t *workspace_bytes);

/*
 * gqa_weighted_pool_kv -- the weighted variant of gqa_mean_pool_kv: each
 * group is a weighted sum of its r heads with caller-given per-head weights,
 * out[n,g,:] = sum_{j<r} weights[g*r + j] * in[n, g*r + j, :] (fp32
 * accumulation in head order). weights[h] = 1/r for every head gives the
 * mean up to rounding.
 * Defines: "Grouped-Query Attention" (llm-arch-kb), section 4 Empirical
 * evidence, the Chinchilla-scale reproduction (groups formed with learned
 * per-head weights rather than the plain mean; learning them is the caller's
 * business).
 *   weights  [H] fp32 DEVICE memory, 4-byte aligned, not overlapping out.
 * Other arguments, layouts and errors as for gqa_mean_pool_kv.
 */
gqa_status gqa_weighted_pool_kv(const void *in, const float *weights, int64_t N, int H, int G, int d_h,
                                gqa_dtype dtype, void *out, hipStream_t stream);

/* Short constant text for a status code. */
const char *gqa_status_string(gqa_status s);

/* Text of the last failure on the calling thread ("" if none): the HIP
 * runtime's message after GQA_ERR_HIP, the failed check otherwise. */
const char *gqa_last_hip_error(void);

/* The same text as gqa_last_hip_error (older name, kept). */
const char *gqa_last_error(void);

/*
 * gqa_release_workspaces -- free every decode workspace the library holds
 * (on every device and stream, including blocks kept alive for captured
 * graphs), after waiting for the devices that hold them to go idle. Graphs
 * captured before this call must not be replayed after it; no other library
 * call may run concurrently. The next decode call allocates afresh.
 */
gqa_status gqa_release_workspaces(void);

/* Library ABI version: 2. */
int gqa_abi_version(void);

/*
 * gqa_debug_checks -- the device range checks of a debug build.
 * libgqa_debug.so is the same library compiled with -DGQA_DEBUG: every
 * kernel checks the index of each global-memory access (cache positions
 * against Tmax, rows against B*H or B*T*H, partial-row slots against the
 * workspace, tile rows against T) and, on a failure, sets a flag and skips
 * the access instead of faulting. This call waits for the current device to
 * go idle, then writes to *flags the flags raised on it since the previous
 * call (bits 0-15 decode and merge kernels, 16-23 prefill, 24-31 pooling;
 * 0: no violation) and clears them; *enabled = 1. In the release library
 * (libgqa.so) the checks are compiled out: *enabled = 0, *flags = 0, and
 * nothing waits. Either pointer may be NULL. GQA_ERR_HIP if the wait or the
 * flag copies fail.
 */
gqa_status gqa_debug_checks(int *enabled, uint32_t *flags);

/*
 * gqa_debug_selftest -- debug library only: queues on `stream` one range
 * check that fails by construction and guards no memory access, so that the
 * next gqa_debug_checks reports bit 31 (pooling word, bit 7). Lets a caller
 * confirm that violations reach the host. GQA_ERR_UNSUPPORTED in the release
 * library (nothing queued).
 */
gqa_status gqa_debug_selftest(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
