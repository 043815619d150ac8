// decode.hip -- GQA decode kernels for gfx950.
//
// Computes, for every sequence b and query head h of group g = h / r,
//   out[b,h,:] = sum_{t < L_b} softmax_t(scale * q[b,h,:] . K[b,t,g,:]) V[b,t,g,:]
// ("Grouped-Query Attention" (llm-arch-kb): section 1 Premise, every cached
// entry is read at a decode step; section 2 Derivation, The grouping; section
// 3 sketch, scaled scores, softmax over keys, times v).
//
// 16-bit design, bf16 or fp16 storage (HBM-bound: every K/V byte is read
// exactly once):
//  * Work partition. The sequences' cache positions are laid end to end
//    (sequence b owns flat positions [pre_b, pre_b + L_b)) and cut into equal
//    pieces of P positions, P = ceil(sum_b L_b / workgroups) rounded up to 32,
//    computed on the device from seqlens. Workgroup k takes flat positions
//    [k P, (k+1) P), whatever sequences they belong to, so ragged batches and
//    single long sequences balance the same way.
//  * One workgroup covers GB adjacent key/value groups of its positions, one
//    group per wave (or WAVES/GB waves per group that share its tiles). With
//    GB = G = 8 every workgroup streams whole contiguous cache rows
//    [t, 0:G, 0:d_h]; a workgroup per group would only touch one 256-byte
//    slice of every 2 KiB row, which concentrates its traffic on a subset of
//    memory channels and makes some groups markedly slower than others.
//  * Within a wave, all r = H/G query heads of its group share every K/V tile:
//    the heads are the N dimension of 16x16x32 bf16 MFMAs.
//  * Scores: S^T[token, head] = K_tile . q^T. K goes from HBM straight into
//    registers in the MFMA A layout (lane = token row, 16-byte chunk of d_h),
//    q sits in registers as the B operand.
//  * The C layout of S^T (lane holds 4 tokens of one head) is already the B
//    operand layout of P^T for O^T = V^T P^T, with tokens as the contraction
//    index, so P never leaves registers.
//  * V is loaded with fully coalesced 16-byte rows, written to a per-wave LDS
//    tile, and read back with ds_read_b64_tr_b16, which delivers 4 consecutive
//    tokens of one d column per lane: the A operand of V^T.
//  * Software pipeline with one register buffer each for K and V: the next
//    tile's K is requested once this tile's scores are computed and its V
//    once this tile's V sits in LDS, so both overlap the softmax and P.V.
//  * K and V rows are read with nontemporal loads where no other workgroup
//    reads them again (one head tile per group): the streaming cache policy
//    raised the achieved bandwidth by 6-7%.
//  * Online softmax in base 2 (the fp32 scores are multiplied by
//    scale*log2(e)); row maxima use two VALU lane swaps per tile (not LDS
//    permutes, which would wait behind the tile's V^T reads).
//  * Waves that share a group (WAVES/GB > 1) combine their softmax states in
//    LDS at the end of each piece, so a piece always leaves the workgroup as
//    one row per head.
//  * A sequence that lies wholly inside one workgroup's piece is written to
//    `out` directly. Otherwise each piece writes a normalised fp32 partial
//    row and its base-2 log-sum-exp, and a second, small kernel merges the
//    partials of every row (the kernel boundary orders the two; no atomics
//    are used).
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

constexpr int kTile = 32;  // positions per wave iteration
constexpr int kPrioMinPositions = 1024;  // slices from this length on use the falling wave priority

template <int D, int NT>
struct TileCfg {
    static constexpr int KS = D / 32;          // MFMA k-steps over d_h
    static constexpr int DT = D / 16;          // 16-wide d tiles of the output
    static constexpr int CH = D / 8;           // 16-byte chunks per row
    static constexpr int VROWS = 64 / CH;      // K or V rows per coalesced load
    static constexpr int VLOADS = kTile / VROWS;  // loads per K or V tile
    static constexpr int LDS_STRIDE = D + 16;  // padded row (elements): 4 rows cover all banks
    static constexpr int HEADS = 16 * NT;
};

template <int D>
struct RowSwz {
    // LDS row swizzles: 16-byte chunk c of tile row r sits at slot c ^ f(r).
    // K: the 16 rows a score fragment read takes at one chunk go to 16
    // different slots (d_h = 128: 16 chunks per row; d_h = 64: 8 chunks, rows
    // of one parity share a bank half).
    static __device__ __forceinline__ int k(int r) { return D >= 128 ? (r & 15) : ((r >> 1) & 7); }
    // V: chunk pairs move together (a transposing read takes 8 bytes of a
    // 32-byte pair); the 8 rows of a half-wave's read go to 8 different pairs.
    static __device__ __forceinline__ int v(int r) { return D >= 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
};

__device__ __forceinline__ u32x4_t load16(const __bf16 *p)
{
    return *reinterpret_cast<const u32x4_t *>(p);
}

// Cache rows read once per call go through nontemporal loads (streaming
// cache policy): measured 5.9 -> 6.6 TB/s for a plain 256 MiB read on this
// chip, and 6-7% off every decode workload with one 16-head tile per group.
// Wider groups (two head tiles, or more head tiles that read the same rows
// from another workgroup) keep the default policy: measured, streaming loads
// made them up to 22% slower.
template <bool STREAM>
__device__ __forceinline__ u32x4_t load16_kv(const __bf16 *p)
{
    if constexpr (STREAM)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    else
        return *reinterpret_cast<const u32x4_t *>(p);
}

// The cache positions one decode step reads for a sequence: [lo, lo + n).
// L0 = clamp(seqlens[b], 0, Tmax). With append, a sequence whose cache is not
// full gains the new token at position L0 (read from k_new/v_new, written to
// the cache), so it holds L = L0 + 1 positions; a full one keeps Tmax. A
// sliding window keeps the `window` newest positions: lo = max(0, L - window).
// The appended token, when there is one, is the last of the n positions.
struct Span {
    int lo, n;
    bool appended;
};

__device__ __forceinline__ Span seq_span(int32_t s, int Tmax, int append, int window)
{
    const int L0 = clamp_len(s, Tmax);
    const bool app = append && L0 < Tmax;
    const int L = L0 + (app ? 1 : 0);
    const int lo = (window > 0 && L > window) ? L - window : 0;
    return {lo, L - lo, app};
}

// Flat-position partition shared by the decode and merge kernels (both must
// compute identical values): total positions and the piece length P. Every
// non-empty sequence is preceded by `startup` virtual positions, the cost of
// starting a piece (first round trips, the combine at its end) in units of
// positions: a workgroup whose range holds the start of a sequence then takes
// that many fewer real positions, which evens out the workgroups' finishing
// times. A negative `startup` (the narrow kernel's default plan) asks for a
// charge of -startup positions only where it leaves the tile-rounded slice
// length unchanged, so that it never costs a workgroup: on the ragged
// Llama-2-70B batch (P = 1152, 29 positions of rounding slack per slice) the
// one-tile charge took 193.4 to 190.9 us; a uniform batch whose spans fill
// the slices exactly (the Llama-3-8B layer, P = 256) keeps none. The host
// guarantees B * (Tmax + |startup|) < 2^31, so position counts fit in 32
// bits. `n_first` is this lane's span length among the first 64 sequences
// (0 past B); the caller has read those lengths already and keeps them for
// its walk. Every lane of the wave must call this (the counts use ballots).
struct Partition {
    int64_t total;
    int64_t P;
    int startup;  // the charge in effect
};

__device__ __forceinline__ int with_startup(int n, int startup)
{
    return n > 0 ? n + startup : 0;
}

// Slice length for `tot` flat positions over nwg workgroups, in whole tiles
// (32-bit: flat positions stay below 2^31).
__device__ __forceinline__ uint32_t slice_positions(uint32_t tot, uint32_t nwg)
{
    uint32_t P = (tot + nwg - 1) / nwg;
    P = ((P + kTile - 1) / kTile) * kTile;
    return P < (uint32_t)kTile ? (uint32_t)kTile : P;
}

__device__ __forceinline__ Partition make_partition(int n_first, const int32_t *seqlens, int B, int Tmax, int append,
                                                    int window, int nwg, int fixed_P, int startup, int lane)
{
    const int c0 = startup < 0 ? 0 : startup;
    int part = with_startup(n_first, c0);
    int nnz = __popcll(__ballot(n_first > 0));  // non-empty sequences (wave-uniform: every lane runs every chunk)
    for (int i0 = 64; i0 < B; i0 += 64) {
        const int i = i0 + lane;
        const int n = i < B ? seq_span(seqlens[i], Tmax, append, window).n : 0;
        part += with_startup(n, c0);
        nnz += __popcll(__ballot(n > 0));
    }
    int64_t tot = wave_total(part);
    int eff = c0;
    int64_t P;
    if (fixed_P > 0) {
        P = fixed_P;
    } else {
        P = slice_positions((uint32_t)tot, (uint32_t)nwg);
        if (startup < 0) {
            const int64_t charged = tot + (int64_t)(-startup) * nnz;
            if (slice_positions((uint32_t)charged, (uint32_t)nwg) == P) {
                tot = charged;
                eff = -startup;
            }
        }
    }
    return {tot, P, eff};
}

// Lanes (sequences of a 64-sequence chunk starting at flat position `pre`,
// inclusive scan `incl` of their lengths with startup positions, real length
// L) whose real positions meet [lo, hi), as a wave-uniform bit mask. The
// set bits form one contiguous run.
__device__ __forceinline__ uint64_t overlapping(int64_t pre, int incl, int L, int64_t lo, int64_t hi)
{
    const int64_t first = pre + incl - L;  // first real position of the lane's sequence
    return __ballot(L > 0 && first < hi && first + L > lo);
}

// One wave's work on one piece: positions [ta, tb) of sequence b for the
// heads [h0, h0 + nheads) of group g. The wave takes tiles ta + sub*32,
// ta + (sub + WPG)*32, ...; with WPG > 1 the group's waves then combine
// their states (every wave of the workgroup must call this for the same
// pieces: the combine has workgroup barriers). Writes the finished rows to
// `out` when `whole`, else a normalised partial row per head and its base-2
// log-sum-exp. `vl_all` and `kl_all` are the workgroup's V-tile and K-tile
// LDS, one tile of each per wave.
//
// `slice_done` is the number of positions of the workgroup's slice before this
// piece, `slice_len` the slice's length (for the wave priority below).
//
// APPEND: position t_new (relative to the span, or -1) is the appended token:
// its rows come from knew_row/vnew_row (this group's slice of k_new, v_new)
// and, when store_new, are written to the cache at that position.
template <typename T, int D, int NT, int WPG, bool APPEND>
__device__ __forceinline__ void decode_piece(const __bf16 *__restrict__ q, __bf16 *kc, __bf16 *vc, int b, int g,
                                             int h0, int nheads, int t_off, int ta, int tb, int t_new,
                                             const __bf16 *knew_row, const __bf16 *vnew_row, bool store_new,
                                             bool whole, int H, int G, int Tmax, int sub, float scale_log2,
                                             __bf16 *vl_all, __bf16 *kl_all, __bf16 *__restrict__ out, float *__restrict__ part_row,
                                             float *__restrict__ lse_row, int lane, bool store_ok, int slice_done,
                                             int slice_len)
{
    const int wave = threadIdx.x >> 6;
    __bf16 *vl = vl_all + wave * kTile * TileCfg<D, NT>::LDS_STRIDE;  // this wave's V tile
    __bf16 *kl = kl_all + wave * kTile * D;                            // this wave's K tile (swizzled)
    using C = TileCfg<D, NT>;
    const int col = lane & 15, kb = lane >> 4;
    const int64_t row0 = (int64_t)b * H + h0;

    // q as the MFMA B operand: column = head, k = d chunk (4*s + kb).
    bf16x8_t qf[NT][C::KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int hh = nt * 16 + col;
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            u32x4_t v = {0, 0, 0, 0};
            if (hh < nheads && GQA_IN_RANGE(h0 + hh, H, 1))
                v = load16(q + (row0 + hh) * D + (s * 4 + kb) * 8);
            qf[nt][s] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    const int64_t tok_stride = (int64_t)G * D;
    __bf16 *kbase = kc + (((int64_t)b * Tmax + t_off) * G + g) * D;  // span position 0
    __bf16 *vbase = vc + (((int64_t)b * Tmax + t_off) * G + g) * D;

    float m_run[NT], l_run[NT];
    f32x4_t acc[NT][C::DT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
            acc[nt][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }

    // Loads are unconditional: rows past the piece are clamped to its last
    // row, and the values they bring are discarded below (scores set to -inf,
    // V rows replaced by zeros). Keeping per-lane branches away from loads
    // lets the compiler wait for exactly the data it needs.
    //
    // K and V both load whole row slices (the 64 lanes of one instruction
    // cover 64/CH rows x the group's d_h*2 bytes) and both pass through this
    // wave's LDS. K loaded straight into the MFMA A layout would take 16 rows
    // x 64 bytes per instruction; measured on a plain read of this layout,
    // that pattern streamed 6-8% slower (6.41 against 6.80 TB/s), and moving
    // K through LDS took the ragged Llama-2-70B batch from 203.2 to 196.2 us.
    const int t_last = tb - 1;
    auto load_k = [&](int t0, u32x4_t (&kr)[C::VLOADS]) {
#pragma unroll
        for (int i = 0; i < C::VLOADS; ++i) {
            const int t = min(t0 + i * C::VROWS + lane / C::CH, t_last);
            const __bf16 *src = kbase + t * tok_stride;
            if constexpr (APPEND)
                src = (t == t_new) ? knew_row : src;
            const bool ok = (APPEND && t == t_new) || GQA_IN_RANGE(t_off + t, Tmax, 0);
            kr[i] = ok ? load16_kv<NT == 1>(src + (lane % C::CH) * 8) : (u32x4_t){0, 0, 0, 0};
        }
    };
    auto load_v = [&](int t0, u32x4_t (&vr)[C::VLOADS]) {
#pragma unroll
        for (int i = 0; i < C::VLOADS; ++i) {
            const int t = min(t0 + i * C::VROWS + lane / C::CH, t_last);
            const __bf16 *src = vbase + t * tok_stride;
            if constexpr (APPEND)
                src = (t == t_new) ? vnew_row : src;
            const bool ok = (APPEND && t == t_new) || GQA_IN_RANGE(t_off + t, Tmax, 0);
            vr[i] = ok ? load16_kv<NT == 1>(src + (lane % C::CH) * 8) : (u32x4_t){0, 0, 0, 0};
        }
    };

    // Software pipeline with one K and one V register buffer: the next K is
    // requested as soon as this tile's scores have consumed K, the next V as
    // soon as this tile's V is in LDS; both arrive while the softmax and P.V
    // of this tile run. The K/V pointers are deliberately not __restrict__
    // (with it the loads count as invariant and get moved across the fences
    // below), and the scheduling barriers keep each request at its place.
    // (Two tiles in flight per wave measured slower, also for the waves of
    // 32-head tiles that have a SIMD to themselves.)
    const int stride = WPG * kTile;
    int t0 = ta + sub * kTile;
    const bool any_tile = t0 < tb;  // wave-uniform
    u32x4_t kbuf[C::VLOADS], vbuf[C::VLOADS];
    if (any_tile) {
        load_k(t0, kbuf);
        load_v(t0, vbuf);
    }
    auto tile = [&](u32x4_t (&kbf)[C::VLOADS], u32x4_t (&vbf)[C::VLOADS], const int tc)
                    __attribute__((always_inline)) {
        const int tn = tc + stride;  // the tile these buffers take next

        // K tile into this wave's LDS rows, 16-byte chunk c of row r at slot
        // c ^ RowSwz::k(r), then the next K into the freed registers.
#pragma unroll
        for (int i = 0; i < C::VLOADS; ++i) {
            const int tl = i * C::VROWS + lane / C::CH;
            const int c = lane % C::CH;
            *reinterpret_cast<u32x4_t *>(kl + tl * D + ((c ^ RowSwz<D>::k(tl)) * 8)) = kbf[i];
        }
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);
        load_k(tn, kbf);  // clamped prefetch, also past the end
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);

        // S^T = K q^T for two 16-token row tiles; A fragments from LDS.
        f32x4_t st[2][NT];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            bf16x8_t kf[C::KS];
#pragma unroll
            for (int s = 0; s < C::KS; ++s) {
                const int row = mt * 16 + col, ch = s * 4 + kb;
                kf[s] = *reinterpret_cast<const bf16x8_t *>(kl + row * D + ((ch ^ RowSwz<D>::k(row)) * 8));
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < C::KS; ++s)
                    c = mfma16x16x32<T>(kf[s], qf[nt][s], c);
                st[mt][nt] = c;
            }
        }
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);

        // V tile into this wave's LDS rows (natural [token][d] order); rows
        // past the piece become zeros so that p = 0 never meets a NaN.
#pragma unroll
        for (int i = 0; i < C::VLOADS; ++i) {
            const int tl = i * C::VROWS + lane / C::CH;
            const u32x4_t zero = {0, 0, 0, 0};
            *reinterpret_cast<u32x4_t *>(vl + tl * C::LDS_STRIDE + (lane % C::CH) * 8) =
                (tc + tl < tb) ? vbf[i] : zero;
        }
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);
        load_v(tn, vbf);
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);

        // Online softmax (base 2). Lane holds tokens tc + 16*mt + 4*kb + i of head column col.
        bf16x8_t pf[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = tc + mt * 16 + kb * 4 + i;
                    const float x = (t < tb) ? st[mt][nt][i] * scale_log2 : -INFINITY;
                    st[mt][nt][i] = x;
                    mx = fmaxf(mx, x);
                }
            mx = xor_fmax<16>(mx);
            mx = xor_fmax<32>(mx);
            const float m_new = fmaxf(m_run[nt], mx);
            const float alpha = fast_exp2(m_run[nt] - m_new);
            m_run[nt] = m_new;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[mt][nt][i] = fast_exp2(st[mt][nt][i] - m_new);
            pf[nt] = pack8<T>(st[0][nt], st[1][nt]);
            // The denominator sums the same bf16-rounded weights that enter
            // the P.V product, so the output is a convex combination of V rows.
            const u32x4_t pu = __builtin_bit_cast(u32x4_t, pf[nt]);
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                psum += bits_to_f32<T>(pu[j] & 0xffffu) + bits_to_f32<T>(pu[j] >> 16);
            l_run[nt] = l_run[nt] * alpha + psum;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
                acc[nt][dt] *= alpha;
        }

        // O^T += V^T P^T; V^T fragments come from transposing LDS reads.
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            const __bf16 *p0 = vl + (kb * 4 + (col >> 2)) * C::LDS_STRIDE + dt * 16 + (col & 3) * 4;
            const bf16x4_t lo = lds_read_tr16(p0);
            const bf16x4_t hi = lds_read_tr16(p0 + 16 * C::LDS_STRIDE);
            const bf16x8_t vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt][dt] = mfma16x16x32<T>(vf, pf[nt], acc[nt][dt]);
        }

    };
    // Wave priority falls from 3 to 0 as the wave gets through its slice.
    // The two waves that share a SIMD stream different groups of the same
    // positions; with equal priority the older one wins the issue
    // arbitration while memory is saturated, and measured on the ragged
    // Llama-2-70B batch, waves 0-3 finished their slices in 118 us and waves
    // 4-7 in 182 us, the last third of the call running on half the waves.
    // Falling priority keeps the pair together (ends 155 against 165 us):
    // 196.9 -> 193.5 us per call. Slices under kPrioMinPositions keep one
    // priority: on the Llama-3-8B layer (256 positions per slice) the
    // scheme measured 1% slower.
    // (Quarter marks of the slice, relative to this piece's tiles: compares
    // only inside the loop.)
    const bool prio = slice_len >= kPrioMinPositions;
    auto mark = [&](int num) {  // position of the slice's num/4 mark in this piece (clamped to int)
        return (int)min<int64_t>((int64_t)ta - slice_done + (int64_t)slice_len * num / 4, INT32_MAX);
    };
    const int q1 = mark(1), q2 = mark(2), q3 = mark(3);
    if (any_tile) {
        for (;;) {
            if (prio) {
                const int t = __builtin_amdgcn_readfirstlane(t0);
                if (t < q1)
                    __builtin_amdgcn_s_setprio(3);
                else if (t < q2)
                    __builtin_amdgcn_s_setprio(2);
                else if (t < q3)
                    __builtin_amdgcn_s_setprio(1);
                else
                    __builtin_amdgcn_s_setprio(0);
            }
            tile(kbuf, vbuf, t0);
            if (t0 + stride >= tb)
                break;
            t0 += stride;
        }
    }

    // The appended token's rows go from k_new / v_new to the cache, written
    // by one wave of the group after the loop: no wave reads that cache row
    // in this call (its tile loads take the row from k_new / v_new). Stores
    // inside the loop would be conditional, and a store that may or may not
    // have been issued leaves the compiler unsure how many memory operations
    // are outstanding, so it would wait for all of them at every tile.
    if constexpr (APPEND) {
        if (store_new && sub == 0 && t_new >= 0 && lane < C::CH && store_ok &&
            GQA_IN_RANGE(t_off + t_new, Tmax, 2)) {
            const u32x4_t kx = load16(knew_row + lane * 8);
            const u32x4_t vx = load16(vnew_row + lane * 8);
            *reinterpret_cast<u32x4_t *>(kbase + t_new * tok_stride + lane * 8) = kx;
            *reinterpret_cast<u32x4_t *>(vbase + t_new * tok_stride + lane * 8) = vx;
        }
    }

    // Finish: the four lanes of one head column hold disjoint token subsets'
    // weight sums; the accumulator lane holds O^T[dt*16 + 4*kb + i][head].
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        l_run[nt] = xor_add<16>(l_run[nt]);
        l_run[nt] = xor_add<32>(l_run[nt]);
    }
    // Output of one head tile: the finished rows when the piece holds the
    // whole sequence, else a normalised fp32 partial row per head and its
    // base-2 log-sum-exp. Lane (col, kb) holds d = dt*16 + 4*kb + i.
    auto emit = [&](int nt, int dt, const f32x4_t &o, float inv) {
        const int hh = nt * 16 + col;
        if (hh >= nheads || !store_ok)
            return;
        if (whole) {
            const f32x4_t x = o * inv;
            u32x2_t u = {pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3])};
            *reinterpret_cast<u32x2_t *>(out + (row0 + hh) * D + kb * 4 + dt * 16) = u;
        } else {
            *reinterpret_cast<f32x4_t *>(part_row + hh * D + kb * 4 + dt * 16) = o * inv;
        }
    };
    if constexpr (WPG == 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const float inv = l_run[nt] > 0.f ? 1.f / l_run[nt] : 0.f;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
                emit(nt, dt, acc[nt][dt], inv);
            if (!whole && kb == 0 && nt * 16 + col < nheads && store_ok)
                lse_row[nt * 16 + col] = l_run[nt] > 0.f ? m_run[nt] + fast_log2(l_run[nt]) : -INFINITY;
        }
    } else {
        // The WPG waves of this group each hold the softmax state of every
        // WPG-th tile. They are combined here, through the V tiles' LDS
        // (free once every wave has left its loop), into one row per head:
        // each wave publishes its maxima, sums and unnormalised accumulators,
        // then combines every WPG-th d tile of all of them. One partial row
        // per head (or the finished output) leaves the workgroup, not WPG.
        constexpr int REG = kTile * C::LDS_STRIDE / 2;  // floats in one wave's V tile
        constexpr int ML = C::DT * 256;                 // offset of the maxima and sums
        static_assert(ML + 32 <= REG, "a wave's state fits in its V tile");
        float *lds = reinterpret_cast<float *>(vl_all);
        float *mine = lds + wave * REG;
        const float *grp = lds + (wave - sub) * REG;  // the group's first wave
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            __syncthreads();  // every wave is done with its V tile (or the previous head tile)
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
                *reinterpret_cast<f32x4_t *>(mine + dt * 256 + lane * 4) = acc[nt][dt];
            if (kb == 0) {
                mine[ML + col] = m_run[nt];
                mine[ML + 16 + col] = l_run[nt];
            }
            __syncthreads();
            float M = -INFINITY;
#pragma unroll
            for (int j = 0; j < WPG; ++j)
                M = fmaxf(M, grp[j * REG + ML + col]);
            float wj[WPG], L = 0.f;
#pragma unroll
            for (int j = 0; j < WPG; ++j) {
                const float mj = grp[j * REG + ML + col];
                wj[j] = mj == -INFINITY ? 0.f : fast_exp2(mj - M);
                L += wj[j] * grp[j * REG + ML + 16 + col];
            }
            const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                if (dt % WPG != sub)
                    continue;
                f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < WPG; ++j)
                    o += wj[j] * *reinterpret_cast<const f32x4_t *>(grp + j * REG + dt * 256 + lane * 4);
                emit(nt, dt, o, inv);
            }
            if (!whole && sub == 0 && kb == 0 && nt * 16 + col < nheads && store_ok)
                lse_row[nt * 16 + col] = L > 0.f ? M + fast_log2(L) : -INFINITY;
        }
        __syncthreads();  // the next piece's loop refills the V tiles
    }
}

template <typename T, int D, int NT, int WAVES, int GB, bool APPEND>
__global__ void __launch_bounds__(WAVES * 64)
decode_split_kernel(const __bf16 *__restrict__ q, __bf16 *kc, __bf16 *vc, const __bf16 *__restrict__ knew,
                   const __bf16 *__restrict__ vnew, const int32_t *__restrict__ seqlens, int B, int H, int G,
                   int Tmax, int window, int r, int head_tiles, float scale_log2, int nwg, int fixed_P, int startup,
                   __bf16 *__restrict__ out, float *__restrict__ part, float *__restrict__ lse)
{
    constexpr int WPG = WAVES / GB;
    using C = TileCfg<D, NT>;
    __shared__ __attribute__((aligned(16))) __bf16 vlds[WAVES][kTile * C::LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) __bf16 klds[WAVES][kTile * D];

    const int k = blockIdx.x;
    const int gblk = blockIdx.y / head_tiles;
    const int ht = blockIdx.y % head_tiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = gblk * GB + wave / WPG;
    const int sub = wave % WPG;
    const int h0 = g * r + ht * C::HEADS;
    const int nheads = min(C::HEADS, r - ht * C::HEADS);

    // The first 64 lengths are read once, for the partition and the walk.
    Span sp0 = {0, 0, false};
    if (lane < B)
        sp0 = seq_span(seqlens[lane], Tmax, APPEND, window);
    const Partition pt = make_partition(sp0.n, seqlens, B, Tmax, APPEND, window, nwg, fixed_P, startup, lane);
    const int64_t lo = (int64_t)k * pt.P;
    if (lo >= pt.total)
        return;
    const int64_t hi = min(lo + pt.P, pt.total);

    // Walk the sequences overlapping [lo, hi), 64 lengths at a time.
    int64_t pre = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        Span sp = sp0;
        if (b0 > 0) {
            sp = {0, 0, false};
            if (b0 + lane < B)
                sp = seq_span(seqlens[b0 + lane], Tmax, APPEND, window);
        }
        const int Lc = sp.n;
        const int incl = wave_incl_scan(with_startup(Lc, pt.startup));
        const int64_t chunk_total = __builtin_amdgcn_readlane(incl, 63);
        if (pre + chunk_total <= lo) {
            pre += chunk_total;
            continue;
        }
        // The sequences of this chunk with positions in [lo, hi): one ballot,
        // then only those (a contiguous run of lanes), in order.
        uint64_t mine = overlapping(pre, incl, Lc, lo, hi);
        while (mine) {
            const int i = __builtin_ctzll(mine);  // wave-uniform
            mine &= mine - 1;
            const int L = __builtin_amdgcn_readlane(Lc, i);
            // first real position of sequence b0 + i in the flat space
            const int64_t pre_b = pre + __builtin_amdgcn_readlane(incl, i) - L;
            const int b = b0 + i;
            const int ta = (int)max<int64_t>(lo - pre_b, 0);
            const int tb = (int)min<int64_t>(hi - pre_b, L);
            const bool whole = ta == 0 && tb == L;
            const int64_t piece = (int64_t)k + b;
            // partial layout [piece][head][d], log-sum-exp [piece][head]
            const int64_t slot = piece * H + h0;
            const int lo_b = __builtin_amdgcn_readlane(sp.lo, i);
            // The appended token is the span's last position, so only the piece
            // that ends there holds it. An earlier piece's last tile can reach
            // past the piece end onto that position with clamped (older) rows
            // in its lanes, and must neither select nor store the new row.
            const int t_new =
                (APPEND && __builtin_amdgcn_readlane((int)sp.appended, i) && tb == L) ? L - 1 : -1;
            const int64_t new_off = ((int64_t)b * G + g) * D;
            // (debug builds: the piece's sequence, group, heads and partial
            // rows; a failure skips its stores, never its barriers)
            const bool store_ok = GQA_IN_RANGE(b, B, 4) && GQA_IN_RANGE(g, G, 4) &&
                                  GQA_IN_RANGE(h0 + nheads - 1, H, 4) &&
                                  (whole || GQA_IN_RANGE(slot + nheads - 1, (int64_t)(nwg + B) * H, 5));
            decode_piece<T, D, NT, WPG, APPEND>(q, kc, vc, b, g, h0, nheads, lo_b, ta, tb, t_new, knew + new_off,
                                             vnew + new_off, ht == 0, whole, H, G, Tmax, sub, scale_log2,
                                             &vlds[0][0], &klds[0][0], out, part + slot * D, lse + slot, lane, store_ok,
                                             (int)(max<int64_t>(pre_b, lo) - lo), (int)(hi - lo));
        }
        if (pre + chunk_total >= hi)
            return;
        pre += chunk_total;
    }
}

// ---------------------------------------------------------------------------
// Wide groups: 33 to 64 query heads per key/value head (multi-query attention
// at 64 heads is the common case). The narrow kernel above gives such a group
// several workgroups that each pull the same rows through their compute unit.
// Here one 8-wave workgroup per (slice, group) streams the group's K/V rows
// into LDS once, with direct-to-LDS loads, and every wave reads them there:
//  * waves form 4 head tiles (16 heads each) x 2 position phases; a step
//    covers 64 positions, 32 per phase;
//  * the stages (K and V of one step, 32 KiB at d_h = 128) form a ring of
//    four buffers, and the loads run three steps ahead, so about 96 KiB per
//    compute unit are in flight while a step is computed; one barrier per
//    step publishes the stage and frees the buffer the next load reuses;
//    every row is read once, with the nontemporal cache policy;
//  * the rows of a stage are swizzled by 16-byte chunk so that the score
//    fragment reads (16 rows at one chunk, 16-byte reads) and the
//    transposing V reads (8 rows x 32 bytes per half-wave) spread over all
//    LDS banks; the buffer range of each stage ends at the piece's last
//    position, so rows past it arrive as zeros;
//  * at the end of a piece the second phase of each head tile hands its
//    softmax state to the first through LDS, which writes the finished rows
//    or one partial row per head.

// LDS chunk swizzles of a stage row r (16-byte chunk c sits at slot c ^ f(r)).

constexpr int kWideWaves = 8;
constexpr int kWideHeadTiles = 4;                         // 16-head tiles per workgroup
constexpr int kWidePhases = kWideWaves / kWideHeadTiles;  // position phases
constexpr int kWideRows = kWidePhases * kTile;            // positions per step
constexpr int kWideRing = 4;                              // stage buffers; loads run kWideRing - 1 steps ahead
constexpr float kWideLazy = 8.f;                          // log2 headroom before the softmax reference moves

// s_waitcnt with vmcnt(n) (n < 64), expcnt and lgkmcnt left free.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for data exchanged through LDS only: this wave's LDS
// operations complete (lgkmcnt(0)), then s_barrier. Unlike __syncthreads()
// it carries no release fence for global memory, which would wait for every
// outstanding vector load (vmcnt(0)), including the direct-to-LDS loads of
// the stages still in flight; the caller waits for the stages it needs.
__device__ __forceinline__ void lds_barrier()
{
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt free
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

template <typename T, int D, bool APPEND>
__global__ void __launch_bounds__(kWideWaves * 64)
decode_wide_kernel(const __bf16 *__restrict__ q, __bf16 *kc, __bf16 *vc, const __bf16 *__restrict__ knew,
                   const __bf16 *__restrict__ vnew, const int32_t *__restrict__ seqlens, int B, int H, int G,
                   int Tmax, int window, int r, float scale_log2, int nwg, int fixed_P, int startup,
                   __bf16 *__restrict__ out,
                   float *__restrict__ part, float *__restrict__ lse)
{
    constexpr int KS = D / 32, DT = D / 16, CH = D / 8;
    constexpr int RPI = 64 / CH;                        // stage rows one load instruction fills
    constexpr int NI = kWideRows / (RPI * kWideWaves);  // load instructions per wave per tensor
    static_assert(NI >= 1 && kWideRows % (RPI * kWideWaves) == 0, "stage rows split evenly over the waves");
    constexpr int TILE = kWideRows * D;  // elements of one stage tensor
    using SW = RowSwz<D>;
    // Separate arrays: the compiler then knows the loads into one buffer do
    // not touch the buffer being read.
    __shared__ __attribute__((aligned(256))) __bf16 K0[TILE];
    __shared__ __attribute__((aligned(256))) __bf16 K1[TILE];
    __shared__ __attribute__((aligned(256))) __bf16 K2[TILE];
    __shared__ __attribute__((aligned(256))) __bf16 K3[TILE];
    __shared__ __attribute__((aligned(256))) __bf16 V0[TILE];
    __shared__ __attribute__((aligned(256))) __bf16 V1[TILE];
    __shared__ __attribute__((aligned(256))) __bf16 V2[TILE];
    __shared__ __attribute__((aligned(256))) __bf16 V3[TILE];
    auto kbuf = [&](auto i) -> __bf16 * {
        constexpr int n = decltype(i)::value;
        if constexpr (n == 0)
            return K0;
        else if constexpr (n == 1)
            return K1;
        else if constexpr (n == 2)
            return K2;
        else
            return K3;
    };
    auto vbuf = [&](auto i) -> __bf16 * {
        constexpr int n = decltype(i)::value;
        if constexpr (n == 0)
            return V0;
        else if constexpr (n == 1)
            return V1;
        else if constexpr (n == 2)
            return V2;
        else
            return V3;
    };

    const int k = blockIdx.x;
    const int g = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ht = wave % kWideHeadTiles, ph = wave / kWideHeadTiles;
    const int col = lane & 15, kb = lane >> 4;
    const int h0 = g * r + ht * 16;
    const int nheads = min(16, r - ht * 16);  // <= 0: a tile past the group (r <= 48)
    const int64_t tok = (int64_t)G * D;      // elements per cache position
    const int tok_bytes = G * D * 2;
    // Per-lane load offsets: instruction u of wave w fills stage rows
    // (u * waves + w) * RPI + lane / CH, slot lane % CH, so it fetches the
    // global chunk the swizzle puts in that slot; the swizzle of those rows
    // does not depend on u.
    const int drow = wave * RPI + lane / CH;
    const int dslot = lane % CH;
    const int voff_k = drow * tok_bytes + g * D * 2 + ((dslot ^ SW::k(drow)) * 16);
    const int voff_v = drow * tok_bytes + g * D * 2 + ((dslot ^ SW::v(drow)) * 16);
    const int ustep = kWideWaves * RPI * tok_bytes;

    // LDS element indices of this lane's fragment reads, the same in every
    // stage: K (A operand of S^T = K q^T) at row 32*ph + 16*mt + col, chunk
    // 4*s + kb; V^T (A operand of O^T = V^T P^T) at rows 32*ph + 4*kb +
    // col/4 and 16 rows on, 4 values from column 16*dt + 4*(col%4). Each read
    // is addressed as stage array + index, with the index opaque to the
    // compiler: it then still knows which LDS array a read touches (through a
    // longer chain of pointer arithmetic it loses track and waits for every
    // load in flight into any stage before the read).
    int kidx[2][KS], vidx[DT][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int rr = mt * 16 + col;
            kidx[mt][s] = (ph * kTile + rr) * D + (((s * 4 + kb) ^ SW::k(rr)) * 8);
            asm("" : "+v"(kidx[mt][s]));
        }
    {
        const int vr = kb * 4 + (col >> 2);
        const int vc0 = (col & 3) >> 1, vhalf = (col & 1) * 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            vidx[dt][0] = (ph * kTile + vr) * D + (((2 * dt + vc0) ^ SW::v(vr)) * 8) + vhalf;
            vidx[dt][1] = vidx[dt][0] + 16 * D;
            asm("" : "+v"(vidx[dt][0]), "+v"(vidx[dt][1]));
        }
    }

    Span sp0 = {0, 0, false};
    if (lane < B)
        sp0 = seq_span(seqlens[lane], Tmax, APPEND, window);
    const Partition pt = make_partition(sp0.n, seqlens, B, Tmax, APPEND, window, nwg, fixed_P, startup, lane);
    const int64_t lo = (int64_t)k * pt.P;
    if (lo >= pt.total)
        return;  // the whole workgroup: lo is uniform
    const int64_t hi = min(lo + pt.P, pt.total);

    int64_t pre = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        Span sp = sp0;
        if (b0 > 0) {
            sp = {0, 0, false};
            if (b0 + lane < B)
                sp = seq_span(seqlens[b0 + lane], Tmax, APPEND, window);
        }
        const int Lc = sp.n;
        const int incl = wave_incl_scan(with_startup(Lc, pt.startup));
        const int64_t chunk_total = __builtin_amdgcn_readlane(incl, 63);
        if (pre + chunk_total <= lo) {
            pre += chunk_total;
            continue;
        }
        // The sequences of this chunk with positions in [lo, hi): one ballot,
        // then only those (a contiguous run of lanes), in order.
        uint64_t mine = overlapping(pre, incl, Lc, lo, hi);
        while (mine) {
            const int i = __builtin_ctzll(mine);  // wave-uniform
            mine &= mine - 1;
            const int L = __builtin_amdgcn_readlane(Lc, i);
            // first real position of sequence b0 + i in the flat space
            const int64_t pre_b = pre + __builtin_amdgcn_readlane(incl, i) - L;
            const int b = b0 + i;
            const int ta = (int)max<int64_t>(lo - pre_b, 0);
            const int tb = (int)min<int64_t>(hi - pre_b, L);
            const bool whole = ta == 0 && tb == L;
            const int64_t slot = ((int64_t)k + b) * H + h0;
            const int t_off = __builtin_amdgcn_readlane(sp.lo, i);
            // only the piece that ends at the span end holds the appended token
            const int t_new = (APPEND && __builtin_amdgcn_readlane((int)sp.appended, i) && tb == L) ? L - 1 : -1;
            const __bf16 *knew_row = knew + ((int64_t)b * G + g) * D;
            const __bf16 *vnew_row = vnew + ((int64_t)b * G + g) * D;
            const __bf16 *kseq = kc + ((int64_t)b * Tmax + t_off) * tok;  // span position 0, every group
            const __bf16 *vseq = vc + ((int64_t)b * Tmax + t_off) * tok;
            const int64_t row0 = (int64_t)b * H + h0;

            // q as the MFMA B operand: column = head, k = d chunk (4*s + kb).
            bf16x8_t qf[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u32x4_t v = {0, 0, 0, 0};
                if (col < nheads && GQA_IN_RANGE(row0 + col, (int64_t)B * H, 6))
                    v = *reinterpret_cast<const u32x4_t *>(q + (row0 + col) * D + (s * 4 + kb) * 8);
                qf[s] = __builtin_bit_cast(bf16x8_t, v);
            }
            float m_run = -INFINITY, l_run = 0.f;
            f32x4_t acc[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                acc[dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            // The appended token's rows, read before the stage loads so that
            // no other vector load sits between them in the loop.
            u32x4_t knew_reg = {0, 0, 0, 0}, vnew_reg = {0, 0, 0, 0};
            if constexpr (APPEND) {
                if (t_new >= 0 && lane < CH) {
                    knew_reg = *reinterpret_cast<const u32x4_t *>(knew_row + lane * 8);
                    vnew_reg = *reinterpret_cast<const u32x4_t *>(vnew_row + lane * 8);
                }
            }

            const int nsteps = (tb - ta + kWideRows - 1) / kWideRows;
            // Stage j (positions ta + 64 j ...) into buffer j % kWideRing:
            // every wave issues its share of the direct-to-LDS loads; rows at
            // or past tb read as zeros.
            auto load_stage = [&](auto B_, int j) {
                const int t0 = ta + j * kWideRows;
                const int nrec = min(kWideRows, tb - t0) * tok_bytes;
                if (GQA_IN_RANGE(t_off + t0, Tmax, 7) && GQA_IN_RANGE(t_off + t0 + min(kWideRows, tb - t0) - 1, Tmax, 7)) {
                    buffer_rows_to_lds<NI, kCpolNT>(kseq + (int64_t)t0 * tok, nrec, kbuf(B_) + wave * 512,
                                                    kWideWaves * 512, voff_k, ustep);
                    buffer_rows_to_lds<NI, kCpolNT>(vseq + (int64_t)t0 * tok, nrec, vbuf(B_) + wave * 512,
                                                    kWideWaves * 512, voff_v, ustep);
                }
            };
            // This wave's 32 rows of stage j: positions t0 + 32*ph + [0, 32).
            auto compute = [&](const __bf16 *Kc, const __bf16 *Vc, int j) __attribute__((always_inline)) {
                const int tc = ta + j * kWideRows + ph * kTile;
                if (tc >= tb || nheads <= 0)
                    return;  // wave-uniform
                f32x4_t st[2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    st[mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const bf16x8_t kf =
                            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(Kc + kidx[mt][s]));
                        st[mt] = mfma16x16x32<T>(kf, qf[s], st[mt]);
                    }
                }
                // Online softmax in base 2; lane holds positions tc + 16*mt +
                // 4*kb + i of head col. Only a tile that crosses the piece end
                // is masked. The reference m_run moves lazily, only when a
                // head's maximum exceeds it by more than 2^kLazy, so most
                // steps skip rescaling the accumulators; probabilities stay
                // below 2^kLazy (exact in real arithmetic).
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    st[mt] *= scale_log2;
                if (tc + kTile > tb) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (tc + mt * 16 + kb * 4 + i >= tb)
                                st[mt][i] = -INFINITY;
                }
                float mx = fmaxf(fmaxf(fmaxf(st[0][0], st[0][1]), fmaxf(st[0][2], st[0][3])),
                                 fmaxf(fmaxf(st[1][0], st[1][1]), fmaxf(st[1][2], st[1][3])));
                mx = xor_fmax<16>(mx);
                mx = xor_fmax<32>(mx);
                const bool move = mx > m_run + kWideLazy;  // m_run = -inf: the first tile moves it
                if (__any(move)) {
                    const float m_new = move ? mx : m_run;
                    const float alpha = fast_exp2(m_run - m_new);
                    m_run = m_new;
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        acc[dt] *= alpha;
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        st[mt][i] = fast_exp2(st[mt][i] - m_run);
                const bf16x8_t pf = pack8<T>(st[0], st[1]);
                const u32x4_t pu = __builtin_bit_cast(u32x4_t, pf);
                float psum = l_run;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    psum = add_pair<T>(pu[jj], psum);
                l_run = psum;
                // O^T += V^T P^T, V^T fragments by transposing reads
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x4_t vlo = lds_read_tr16(Vc + vidx[dt][0]);
                    const bf16x4_t vhi = lds_read_tr16(Vc + vidx[dt][1]);
                    const bf16x8_t vf = __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[dt] = mfma16x16x32<T>(vf, pf, acc[dt]);
                }
            };
            // Step j on buffer B_ = j % kWideRing: wait for this wave's loads
            // of stage j (the loads of the up to two later stages stay in
            // flight), put the appended token's row in place, publish the
            // stage with the barrier (which also frees buffer (j - 1) % ring,
            // read by step j - 1), refill that buffer with stage j + 3, and
            // compute.
            auto step = [&](auto B_, int j) __attribute__((always_inline)) {
                constexpr int b_ = decltype(B_)::value;
                const int ahead = min(kWideRing - 2, nsteps - 1 - j);  // stages issued after stage j
                if (ahead >= 2)
                    wait_vmcnt<4 * NI>();
                else if (ahead == 1)
                    wait_vmcnt<2 * NI>();
                else
                    wait_vmcnt<0>();
                if constexpr (APPEND) {
                    // The wave whose load instruction filled the appended
                    // token's stage row replaces it with k_new / v_new.
                    const int rn = t_new - (ta + j * kWideRows);
                    if (t_new >= 0 && rn >= 0 && rn < kWideRows && (rn / RPI) % kWideWaves == wave && lane < CH) {
                        *reinterpret_cast<u32x4_t *>(kbuf(B_) + rn * D + ((lane ^ SW::k(rn)) * 8)) = knew_reg;
                        *reinterpret_cast<u32x4_t *>(vbuf(B_) + rn * D + ((lane ^ SW::v(rn)) * 8)) = vnew_reg;
                    }
                }
                lds_barrier();
                if (j + kWideRing - 1 < nsteps)
                    load_stage(Ic<(b_ + kWideRing - 1) % kWideRing>{}, j + kWideRing - 1);
                compute(kbuf(B_), vbuf(B_), j);
            };

            load_stage(Ic<0>{}, 0);
            if (nsteps > 1)
                load_stage(Ic<1>{}, 1);
            if (nsteps > 2)
                load_stage(Ic<2>{}, 2);
            for (int j = 0;; j += kWideRing) {
                step(Ic<0>{}, j);
                if (j + 1 >= nsteps)
                    break;
                step(Ic<1>{}, j + 1);
                if (j + 2 >= nsteps)
                    break;
                step(Ic<2>{}, j + 2);
                if (j + 3 >= nsteps)
                    break;
                step(Ic<3>{}, j + 3);
                if (j + 4 >= nsteps)
                    break;
            }

            // The appended token goes from k_new / v_new to the cache; no
            // workgroup reads that cache row in this call.
            if constexpr (APPEND) {
                if (t_new >= 0 && wave == 0 && lane < CH && GQA_IN_RANGE(b, B, 4) &&
                    GQA_IN_RANGE(t_off + t_new, Tmax, 2)) {
                    *reinterpret_cast<u32x4_t *>(kc + ((int64_t)b * Tmax + t_off + t_new) * tok + g * D + lane * 8) =
                        knew_reg;
                    *reinterpret_cast<u32x4_t *>(vc + ((int64_t)b * Tmax + t_off + t_new) * tok + g * D + lane * 8) =
                        vnew_reg;
                }
            }

            // The second phase of each head tile hands its state to the first
            // through LDS (stage buffers, free once every wave has left the
            // loop): accumulators into K0 / K1, maxima and sums into V0.
            l_run = xor_add<16>(l_run);
            l_run = xor_add<32>(l_run);
            static_assert(2 * DT * 256 * 4 <= TILE * 2, "two waves' accumulators fit in one K stage");
            float *accs = reinterpret_cast<float *>((ht >> 1) ? K1 : K0) + (ht & 1) * DT * 256;
            float *stat = reinterpret_cast<float *>(V0) + ht * 32;
            __syncthreads();  // every wave is done with the stages
            if (ph == 1) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    *reinterpret_cast<f32x4_t *>(accs + dt * 256 + lane * 4) = acc[dt];
                if (kb == 0) {
                    stat[col] = m_run;
                    stat[16 + col] = l_run;
                }
            }
            __syncthreads();
            if (ph == 0 && col < nheads) {
                const float m1 = stat[col], l1 = stat[16 + col];
                const float M = fmaxf(m_run, m1);
                const float w0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - M);
                const float w1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
                const float Ls = w0 * l_run + w1 * l1;
                const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const f32x4_t o = w0 * acc[dt] + w1 * *reinterpret_cast<const f32x4_t *>(accs + dt * 256 + lane * 4);
                    if (whole) {
                        const f32x4_t x = o * inv;
                        u32x2_t u = {pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3])};
                        if (GQA_IN_RANGE(row0 + col, (int64_t)B * H, 8))
                            *reinterpret_cast<u32x2_t *>(out + (row0 + col) * D + kb * 4 + dt * 16) = u;
                    } else if (GQA_IN_RANGE(slot + col, (int64_t)(nwg + B) * H, 8)) {
                        *reinterpret_cast<f32x4_t *>(part + (slot + col) * D + kb * 4 + dt * 16) = o * inv;
                    }
                }
                if (!whole && kb == 0 && GQA_IN_RANGE(slot + col, (int64_t)(nwg + B) * H, 8))
                    lse[slot + col] = Ls > 0.f ? M + fast_log2(Ls) : -INFINITY;
            }
            __syncthreads();  // the next piece's loads refill the stages
        }
        if (pre + chunk_total >= hi)
            return;
        pre += chunk_total;
    }
}

// Merge of the partial rows. Workgroup = (block of 4 row items, sequence b):
// its 256 threads compute the partition once; each wave then merges one item
// = (head h, NQ*4 consecutive d). Lanes form 64/NQ slot lanes x NQ d-quads:
// slot lane sl takes the row's pieces sl, sl + 64/NQ, ... (U per round) and
// the lanes of a d-quad are combined with shuffles. out = sum_j w_j o_j with
// w_j = 2^(lse_j - M) / sum_j' 2^(lse_j' - M). Also writes the zero rows of
// empty sequences; rows that the decode kernel wrote whole are skipped.
template <typename T, int D, int NQ, int U>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const int32_t *__restrict__ seqlens, int B, int H, int Tmax, int append, int window, int nwg,
                    int fixed_P, int startup, const float *part, const float *lse, __bf16 *__restrict__ out)
{
    constexpr int DCH = 4 * NQ;      // d values per item
    constexpr int NDC = D / DCH;     // items per row
    constexpr int NS = 64 / NQ;      // slot lanes
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.y;
    const int item = blockIdx.x * 4 + wave;
    if (item >= H * NDC)
        return;

    // partition and this sequence's first real flat position, after its
    // startup positions (each wave on its own)
    const int c0 = startup < 0 ? 0 : startup;
    int tot_part = 0, pre_part = 0, L_first = 0, nnz = 0, pre_nnz = 0;  // counts wave-uniform
    for (int i0 = 0; i0 < B; i0 += 64) {
        const int i = i0 + lane;
        const int Li = i < B ? seq_span(seqlens[i], Tmax, append, window).n : 0;
        tot_part += with_startup(Li, c0);
        nnz += __popcll(__ballot(Li > 0));
        pre_nnz += __popcll(__ballot(Li > 0 && i < b));
        if (i < b)
            pre_part += with_startup(Li, c0);
        if (i0 == 0)
            L_first = Li;
    }
    // 32-bit arithmetic: flat positions stay below 2^31 (the host checks
    // B * (Tmax + startup) < 2^31), and the slice length is the same as the
    // decode kernels' (make_partition).
    uint32_t tot = (uint32_t)wave_total(tot_part);
    uint32_t pre0 = (uint32_t)wave_total(pre_part);
    int eff = c0;
    uint32_t P;
    if (fixed_P > 0) {
        P = (uint32_t)fixed_P;
    } else {
        P = slice_positions(tot, (uint32_t)nwg);
        if (startup < 0) {
            const uint32_t charged = tot + (uint32_t)(-startup) * (uint32_t)nnz;
            if (slice_positions(charged, (uint32_t)nwg) == P) {
                tot = charged;
                eff = -startup;
                pre0 += (uint32_t)eff * (uint32_t)pre_nnz;
            }
        }
    }
    const uint32_t pre_b = pre0 + (uint32_t)eff;

    const int h = item / NDC, dc = item % NDC;
    const int sl = lane / NQ, qd = lane % NQ;
    const int d0 = dc * DCH + qd * 4;
    __bf16 *dst = out + ((int64_t)b * H + h) * D + d0;
    const int L = b < 64 ? __builtin_amdgcn_readlane(L_first, b) : seq_span(seqlens[b], Tmax, append, window).n;
    if (L == 0) {
        if (sl == 0 && GQA_IN_RANGE((int64_t)b * H + h, (int64_t)B * H, 10))
            *reinterpret_cast<u32x2_t *>(dst) = (u32x2_t){0, 0};
        return;
    }
    const int64_t k_first = pre_b / P;
    const int64_t k_last = (pre_b + (uint32_t)L - 1) / P;
    if (k_first == k_last)
        return;  // written whole by the decode kernel
    const int nslots = (int)(k_last - k_first + 1);

    float m = -INFINITY, den = 0.f;
    f32x4_t num = {0.f, 0.f, 0.f, 0.f};
    // U slots per lane per round, loads issued together
    for (int j0 = sl; j0 < nslots; j0 += NS * U) {
        float x[U];
        f32x4_t pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(j0 + NS * u, nslots - 1);
            const int64_t idx = (k_first + j + b) * H + h;  // slot of piece k_first + j
            const bool ok = GQA_IN_RANGE(idx, (int64_t)(nwg + B) * H, 9);
            x[u] = ok ? lse[idx] : -INFINITY;
            pv[u] = ok ? *reinterpret_cast<const f32x4_t *>(part + idx * D + d0) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
        }
        // All loads of the round are issued before any is used (the compiler
        // otherwise sinks the last one into the branch that uses it, behind a
        // wait for the first). The partial pointers are not __restrict__ for
        // the same reason: with it the loads may move across this fence.
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (j0 + NS * u >= nslots || x[u] == -INFINITY)
                continue;
            if (x[u] > m) {
                const float f = fast_exp2(m - x[u]);
                den *= f;
                num *= f;
                m = x[u];
            }
            const float w = fast_exp2(x[u] - m);
            den += w;
            num += w * pv[u];
        }
    }
    // combine the slot lanes of each d-quad (lanes qd, qd + NQ, ...), by
    // lane exchanges on the VALU, masks 32, 16, ... down to NQ
    auto over_slots = [&](float x, auto op) {
        if constexpr (NQ <= 32)
            x = op(x, Ic<32>{});
        if constexpr (NQ <= 16)
            x = op(x, Ic<16>{});
        if constexpr (NQ <= 8)
            x = op(x, Ic<8>{});
        if constexpr (NQ <= 4)
            x = op(x, Ic<4>{});
        if constexpr (NQ <= 2)
            x = op(x, Ic<2>{});
        if constexpr (NQ <= 1)
            x = op(x, Ic<1>{});
        return x;
    };
    const auto vmax = [](float x, auto S) { return xor_fmax<decltype(S)::value>(x); };
    const auto vsum = [](float x, auto S) { return xor_add<decltype(S)::value>(x); };
    const float M = over_slots(m, vmax);
    const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
    den *= f;
    num *= f;
    den = over_slots(den, vsum);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        num[e] = over_slots(num[e], vsum);
    if (sl == 0 && GQA_IN_RANGE((int64_t)b * H + h, (int64_t)B * H, 10)) {
        const float inv = 1.f / den;
        u32x2_t u = {pack2<T>(num[0] * inv, num[1] * inv), pack2<T>(num[2] * inv, num[3] * inv)};
        *reinterpret_cast<u32x2_t *>(dst) = u;
    }
}

template <typename T, int D, int NQ, int U>
hipError_t launch_merge(const DecodePlan &p, const DecodeArgs &a)
{
    constexpr int NDC = D / (4 * NQ);
    dim3 grid((unsigned)((a.H * NDC + 3) / 4), (unsigned)a.B);
    decode_merge_kernel<T, D, NQ, U><<<grid, 256, 0, a.stream>>>(a.seqlens, a.B, a.H, a.Tmax, a.knew != nullptr,
                                                          a.window, p.nwg, p.fixed_P, p.startup, a.part, a.lse,
                                                          static_cast<__bf16 *>(a.out));
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_merge_d(const DecodePlan &p, const DecodeArgs &a)
{
    if (p.merge_u == 16) {  // rows of more than 128 pieces: at least 16 slot lanes
        switch (p.merge_nq) {
        case 1: return launch_merge<T, D, 1, 16>(p, a);
        case 2: return launch_merge<T, D, 2, 16>(p, a);
        default: return launch_merge<T, D, 4, 16>(p, a);
        }
    }
    switch (p.merge_nq) {
    case 1: return launch_merge<T, D, 1, 4>(p, a);
    case 2: return launch_merge<T, D, 2, 4>(p, a);
    case 4: return launch_merge<T, D, 4, 4>(p, a);
    case 8: return launch_merge<T, D, 8, 4>(p, a);
    case 16: return launch_merge<T, D, 16, 4>(p, a);
    default: return launch_merge<T, D, (D >= 128 ? 32 : 16), 4>(p, a);
    }
}

// fp32 debug path: one wavefront per (sequence, head); lanes split d_h and the
// wave walks the cache one position at a time with an online softmax.
template <int D>
__global__ void __launch_bounds__(64)
decode_f32_kernel(const float *__restrict__ q, float *kc, float *vc, const float *__restrict__ knew,
                  const float *__restrict__ vnew, const int32_t *__restrict__ seqlens, int H, int G, int Tmax,
                  int append, int window, int r, float scale, float *__restrict__ out)
{
    constexpr int J = D / 64;
    const int64_t row = blockIdx.x;
    const int b = (int)(row / H), h = (int)(row % H);
    const int g = h / r;
    const int lane = threadIdx.x;
    const Span sp = seq_span(seqlens[b], Tmax, append, window);
    const int L = sp.n;
    const int t_new = sp.appended ? L - 1 : -1;  // span position of the appended token
    const int64_t new_off = ((int64_t)b * G + g) * D;
    float qv[J], acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        qv[j] = q[row * D + lane + 64 * j];
        acc[j] = 0.f;
    }
    // Scores and the running maximum in fp64, so that the exponent argument
    // keeps fp32 accuracy at large scores.
    double m = -INFINITY;
    float l = 0.f;
    for (int t = 0; t < L; ++t) {
        if (t != t_new && !GQA_IN_RANGE(sp.lo + t, Tmax, 11))
            continue;
        const int64_t off = (((int64_t)b * Tmax + sp.lo + t) * G + g) * D;
        const float *kp = (t == t_new) ? knew + new_off : kc + off;
        const float *vp = (t == t_new) ? vnew + new_off : vc + off;
        double dot = 0.0;
#pragma unroll
        for (int j = 0; j < J; ++j)
            dot += (double)qv[j] * (double)kp[lane + 64 * j];
        const double s = wave_sum(dot) * (double)scale;
        const double m_new = fmax(m, s);
        const float alpha = expf((float)(m - m_new));
        const float p = expf((float)(s - m_new));
        l = l * alpha + p;
#pragma unroll
        for (int j = 0; j < J; ++j)
            acc[j] = acc[j] * alpha + p * vp[lane + 64 * j];
        m = m_new;
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
        out[row * D + lane + 64 * j] = L > 0 ? acc[j] / l : 0.f;
    if (t_new >= 0 && h % r == 0 && GQA_IN_RANGE(sp.lo + t_new, Tmax, 2)) {  // the group's first head stores the appended token
        const int64_t off = (((int64_t)b * Tmax + sp.lo + t_new) * G + g) * D;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            kc[off + lane + 64 * j] = knew[new_off + lane + 64 * j];
            vc[off + lane + 64 * j] = vnew[new_off + lane + 64 * j];
        }
    }
}

template <typename T, int D, int NT, int WAVES, int GB, bool APPEND>
const void *split_symbol()
{
    return reinterpret_cast<const void *>(&decode_split_kernel<T, D, NT, WAVES, GB, APPEND>);
}

// Wide groups: grid (pieces, groups), 8 waves, then the merge.
template <typename T, int D>
hipError_t launch_wide(const DecodePlan &p, const DecodeArgs &a)
{
    dim3 grid(p.nwg, a.G);
    __bf16 *kc = const_cast<__bf16 *>(static_cast<const __bf16 *>(a.k));
    __bf16 *vc = const_cast<__bf16 *>(static_cast<const __bf16 *>(a.v));
    const __bf16 *q = static_cast<const __bf16 *>(a.q);
    const __bf16 *kn = static_cast<const __bf16 *>(a.knew), *vn = static_cast<const __bf16 *>(a.vnew);
    if (a.knew)
        decode_wide_kernel<T, D, true><<<grid, kWideWaves * 64, 0, a.stream>>>(
            q, kc, vc, kn, vn, a.seqlens, a.B, a.H, a.G, a.Tmax, a.window, p.r, a.scale * kLog2e, p.nwg, p.fixed_P,
            p.startup, static_cast<__bf16 *>(a.out), a.part, a.lse);
    else
        decode_wide_kernel<T, D, false><<<grid, kWideWaves * 64, 0, a.stream>>>(
            q, kc, vc, kn, vn, a.seqlens, a.B, a.H, a.G, a.Tmax, a.window, p.r, a.scale * kLog2e, p.nwg, p.fixed_P,
            p.startup, static_cast<__bf16 *>(a.out), a.part, a.lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_merge_d<T, D>(p, a);
}

// 16-bit storage of type T; the pointers carry its raw bit patterns.
template <typename T, int D, int NT, int WAVES, int GB>
hipError_t launch_split(const DecodePlan &p, const DecodeArgs &a)
{
    dim3 grid(p.nwg, (a.G / GB) * p.head_tiles);
    // The caches are written only when appending (a.knew set).
    __bf16 *kc = const_cast<__bf16 *>(static_cast<const __bf16 *>(a.k));
    __bf16 *vc = const_cast<__bf16 *>(static_cast<const __bf16 *>(a.v));
    const __bf16 *q = static_cast<const __bf16 *>(a.q);
    const __bf16 *kn = static_cast<const __bf16 *>(a.knew), *vn = static_cast<const __bf16 *>(a.vnew);
    if (a.knew)
        decode_split_kernel<T, D, NT, WAVES, GB, true><<<grid, WAVES * 64, 0, a.stream>>>(
            q, kc, vc, kn, vn, a.seqlens, a.B, a.H, a.G, a.Tmax, a.window, p.r, p.head_tiles, a.scale * kLog2e,
            p.nwg, p.fixed_P, p.startup, static_cast<__bf16 *>(a.out), a.part, a.lse);
    else
        decode_split_kernel<T, D, NT, WAVES, GB, false><<<grid, WAVES * 64, 0, a.stream>>>(
            q, kc, vc, kn, vn, a.seqlens, a.B, a.H, a.G, a.Tmax, a.window, p.r, p.head_tiles, a.scale * kLog2e,
            p.nwg, p.fixed_P, p.startup, static_cast<__bf16 *>(a.out), a.part, a.lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_merge_d<T, D>(p, a);
}

// Dispatch over the compiled variants: (d_h, head tiles NT, waves, groups per workgroup GB).
template <typename F>
hipError_t with_variant(const DecodePlan &p, int D, F &&f)
{
#define GQA_VARIANT(DD, NTT, WW, GG)                                       \
    if (D == DD && p.nt == NTT && p.waves == WW && p.gb == GG)             \
        return f.template operator()<DD, NTT, WW, GG>();
#define GQA_VARIANTS(DD)                                                    \
    GQA_VARIANT(DD, 1, 8, 8) GQA_VARIANT(DD, 1, 8, 4) GQA_VARIANT(DD, 1, 8, 2) GQA_VARIANT(DD, 1, 8, 1) \
    GQA_VARIANT(DD, 2, 4, 4) GQA_VARIANT(DD, 2, 4, 2) GQA_VARIANT(DD, 2, 4, 1)
    GQA_VARIANTS(64)
    GQA_VARIANTS(128)
#undef GQA_VARIANTS
#undef GQA_VARIANT
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t decode_blocks_per_cu(const DecodePlan &p, int D, gqa_dtype dtype, bool append, int *blocks)
{
    if (p.wide) {
        const void *f;
        const bool h = dtype == GQA_FP16;
        if (D == 64)
            f = h ? (append ? (const void *)&decode_wide_kernel<_Float16, 64, true>
                            : (const void *)&decode_wide_kernel<_Float16, 64, false>)
                  : (append ? (const void *)&decode_wide_kernel<__bf16, 64, true>
                            : (const void *)&decode_wide_kernel<__bf16, 64, false>);
        else
            f = h ? (append ? (const void *)&decode_wide_kernel<_Float16, 128, true>
                            : (const void *)&decode_wide_kernel<_Float16, 128, false>)
                  : (append ? (const void *)&decode_wide_kernel<__bf16, 128, true>
                            : (const void *)&decode_wide_kernel<__bf16, 128, false>);
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, f, kWideWaves * 64, 0);
    }
    return with_variant(p, D, [&]<int DD, int NTT, int WW, int GG>() {
        const void *f;
        if (dtype == GQA_FP16)
            f = append ? split_symbol<_Float16, DD, NTT, WW, GG, true>()
                       : split_symbol<_Float16, DD, NTT, WW, GG, false>();
        else
            f = append ? split_symbol<__bf16, DD, NTT, WW, GG, true>() : split_symbol<__bf16, DD, NTT, WW, GG, false>();
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, f, WW * 64, 0);
    });
}

hipError_t launch_decode(const DecodePlan &p, const DecodeArgs &a, gqa_dtype dtype)
{
    if (dtype == GQA_FP32) {
        dim3 grid((unsigned)((int64_t)a.B * a.H));
        const float *q = static_cast<const float *>(a.q);
        float *kc = const_cast<float *>(static_cast<const float *>(a.k));
        float *vc = const_cast<float *>(static_cast<const float *>(a.v));
        const float *kn = static_cast<const float *>(a.knew), *vn = static_cast<const float *>(a.vnew);
        const int app = a.knew != nullptr;
        if (a.D == 64)
            decode_f32_kernel<64><<<grid, 64, 0, a.stream>>>(q, kc, vc, kn, vn, a.seqlens, a.H, a.G, a.Tmax, app,
                                                             a.window, p.r, a.scale, static_cast<float *>(a.out));
        else
            decode_f32_kernel<128><<<grid, 64, 0, a.stream>>>(q, kc, vc, kn, vn, a.seqlens, a.H, a.G, a.Tmax, app,
                                                              a.window, p.r, a.scale, static_cast<float *>(a.out));
        return hipGetLastError();
    }
    if (p.wide) {
        if (dtype == GQA_FP16)
            return a.D == 64 ? launch_wide<_Float16, 64>(p, a) : launch_wide<_Float16, 128>(p, a);
        return a.D == 64 ? launch_wide<__bf16, 64>(p, a) : launch_wide<__bf16, 128>(p, a);
    }
    if (dtype == GQA_FP16)
        return with_variant(p, a.D, [&]<int DD, int NTT, int WW, int GG>() {
            return launch_split<_Float16, DD, NTT, WW, GG>(p, a);
        });
    return with_variant(p, a.D, [&]<int DD, int NTT, int WW, int GG>() {
        return launch_split<__bf16, DD, NTT, WW, GG>(p, a);
    });
}

GQA_DEBUG_READER(debug_take_decode)

}  // namespace gqa
