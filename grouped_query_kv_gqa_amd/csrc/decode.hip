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

template <int D, int NT>
struct TileCfg {
    static constexpr int KS = D / 32;          // MFMA k-steps over d_h
    static constexpr int DT = D / 16;          // 16-wide d tiles of the output
    static constexpr int CH = D / 8;           // 16-byte chunks per row
    static constexpr int VROWS = 64 / CH;      // V rows per coalesced load
    static constexpr int VLOADS = kTile / VROWS;
    static constexpr int LDS_STRIDE = D + 16;  // padded row (elements): 4 rows cover all banks
    static constexpr int HEADS = 16 * NT;
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
// compute identical values): total positions and the piece length P. The
// host guarantees B * Tmax < 2^31, so position counts fit in 32 bits.
// `n_first` is this lane's span length among the first 64 sequences (0 past
// B); the caller has read those lengths already and keeps them for its walk.
struct Partition {
    int64_t total;
    int64_t P;
};

__device__ __forceinline__ Partition make_partition(int n_first, const int32_t *seqlens, int B, int Tmax, int append,
                                                    int window, int nwg, int fixed_P, int lane)
{
    int part = n_first;
    for (int i = lane + 64; i < B; i += 64)
        part += seq_span(seqlens[i], Tmax, append, window).n;
    const int64_t tot = wave_total(part);
    int64_t P;
    if (fixed_P > 0) {
        P = fixed_P;
    } else {
        P = (tot + nwg - 1) / nwg;
        P = ((P + kTile - 1) / kTile) * kTile;
        if (P < kTile)
            P = kTile;
    }
    return {tot, P};
}

// One wave's work on one piece: positions [ta, tb) of sequence b for the
// heads [h0, h0 + nheads) of group g. The wave takes tiles ta + sub*32,
// ta + (sub + WPG)*32, ...; with WPG > 1 the group's waves then combine
// their states (every wave of the workgroup must call this for the same
// pieces: the combine has workgroup barriers). Writes the finished rows to
// `out` when `whole`, else a normalised partial row per head and its base-2
// log-sum-exp. `vl_all` is the workgroup's V-tile LDS, one tile per wave.
//
// APPEND: position t_new (relative to the span, or -1) is the appended token:
// its rows come from knew_row/vnew_row (this group's slice of k_new, v_new)
// and, when store_new, are written to the cache at that position.
template <typename T, int D, int NT, int WPG, bool APPEND>
__device__ __forceinline__ void decode_piece(const __bf16 *__restrict__ q, __bf16 *kc, __bf16 *vc, int b, int g,
                                             int h0, int nheads, int t_off, int ta, int tb, int t_new,
                                             const __bf16 *knew_row, const __bf16 *vnew_row, bool store_new,
                                             bool whole, int H, int G, int Tmax, int sub, float scale_log2,
                                             __bf16 *vl_all, __bf16 *__restrict__ out, float *__restrict__ part_row,
                                             float *__restrict__ lse_row, int lane)
{
    const int wave = threadIdx.x >> 6;
    __bf16 *vl = vl_all + wave * kTile * TileCfg<D, NT>::LDS_STRIDE;  // this wave's V tile
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
            if (hh < nheads)
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
    const int t_last = tb - 1;
    auto load_k = [&](int t0, u32x4_t (&kr)[2][C::KS]) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int t = min(t0 + mt * 16 + col, t_last);
            const __bf16 *src = kbase + t * tok_stride;
            if constexpr (APPEND)
                src = (t == t_new) ? knew_row : src;
#pragma unroll
            for (int s = 0; s < C::KS; ++s)
                kr[mt][s] = load16_kv<NT == 1>(src + (s * 4 + kb) * 8);
        }
    };
    auto load_v = [&](int t0, u32x4_t (&vr)[C::VLOADS]) {
#pragma unroll
        for (int i = 0; i < C::VLOADS; ++i) {
            const int t = min(t0 + i * C::VROWS + lane / C::CH, t_last);
            const __bf16 *src = vbase + t * tok_stride;
            if constexpr (APPEND)
                src = (t == t_new) ? vnew_row : src;
            vr[i] = load16_kv<NT == 1>(src + (lane % C::CH) * 8);
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
    u32x4_t kbuf[2][C::KS], vbuf[C::VLOADS];
    if (any_tile) {
        load_k(t0, kbuf);
        load_v(t0, vbuf);
    }
    auto tile = [&](u32x4_t (&kbf)[2][C::KS], u32x4_t (&vbf)[C::VLOADS], const int tc)
                    __attribute__((always_inline)) {
        const int tn = tc + stride;  // the tile these buffers take next

        // S^T = K q^T for two 16-token row tiles.
        f32x4_t st[2][NT];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < C::KS; ++s)
                    c = mfma16x16x32<T>(__builtin_bit_cast(bf16x8_t, kbf[mt][s]), qf[nt][s], c);
                st[mt][nt] = c;
            }
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);
        load_k(tn, kbf);  // clamped prefetch, also past the end
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
    if (any_tile) {
        for (;;) {
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
        if (store_new && sub == 0 && t_new >= 0 && lane < C::CH) {
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
        if (hh >= nheads)
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
            if (!whole && kb == 0 && nt * 16 + col < nheads)
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
            if (!whole && sub == 0 && kb == 0 && nt * 16 + col < nheads)
                lse_row[nt * 16 + col] = L > 0.f ? M + fast_log2(L) : -INFINITY;
        }
        __syncthreads();  // the next piece's loop refills the V tiles
    }
}

template <typename T, int D, int NT, int WAVES, int GB, bool APPEND>
__global__ void __launch_bounds__(WAVES * 64)
decode_split_kernel(const __bf16 *__restrict__ q, __bf16 *kc, __bf16 *vc, const __bf16 *__restrict__ knew,
                   const __bf16 *__restrict__ vnew, const int32_t *__restrict__ seqlens, int B, int H, int G,
                   int Tmax, int window, int r, int head_tiles, float scale_log2, int nwg, int fixed_P,
                   __bf16 *__restrict__ out, float *__restrict__ part, float *__restrict__ lse)
{
    constexpr int WPG = WAVES / GB;
    using C = TileCfg<D, NT>;
    __shared__ __attribute__((aligned(16))) __bf16 vlds[WAVES][kTile * C::LDS_STRIDE];

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
    const Partition pt = make_partition(sp0.n, seqlens, B, Tmax, APPEND, window, nwg, fixed_P, lane);
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
        const int incl = wave_incl_scan(Lc);
        const int64_t chunk_total = __builtin_amdgcn_readlane(incl, 63);
        if (pre + chunk_total <= lo) {
            pre += chunk_total;
            continue;
        }
        const int n = min(64, B - b0);
        for (int i = 0; i < n; ++i) {
            const int L = __builtin_amdgcn_readlane(Lc, i);  // i is wave-uniform
            const int64_t pre_b = pre + __builtin_amdgcn_readlane(incl, i) - L;
            if (pre_b >= hi)
                return;
            if (L == 0 || pre_b + L <= lo)
                continue;
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
            decode_piece<T, D, NT, WPG, APPEND>(q, kc, vc, b, g, h0, nheads, lo_b, ta, tb, t_new, knew + new_off,
                                             vnew + new_off, ht == 0, whole, H, G, Tmax, sub, scale_log2,
                                             &vlds[0][0], out, part + slot * D, lse + slot, lane);
        }
        pre += chunk_total;
    }
}

// Merge of the partial rows. Workgroup = (block of 4 row items, sequence b):
// its 256 threads compute the partition once; each wave then merges one item
// = (head h, NQ*4 consecutive d). Lanes form 64/NQ slot lanes x NQ d-quads:
// slot lane sl takes the row's pieces sl, sl + 64/NQ, ... and the lanes of a
// d-quad are combined with shuffles. out = sum_j w_j o_j with
// w_j = 2^(lse_j - M) / sum_j' 2^(lse_j' - M). Also writes the zero rows of
// empty sequences; rows that the decode kernel wrote whole are skipped.
template <typename T, int D, int NQ>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const int32_t *__restrict__ seqlens, int B, int H, int Tmax, int append, int window, int nwg,
                    int fixed_P, const float *part, const float *lse, __bf16 *__restrict__ out)
{
    constexpr int DCH = 4 * NQ;      // d values per item
    constexpr int NDC = D / DCH;     // items per row
    constexpr int NS = 64 / NQ;      // slot lanes
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.y;
    const int item = blockIdx.x * 4 + wave;
    if (item >= H * NDC)
        return;

    // partition and this sequence's first flat position (each wave on its own)
    int tot_part = 0, pre_part = 0, L_first = 0;
    for (int i = lane; i < B; i += 64) {
        const int Li = seq_span(seqlens[i], Tmax, append, window).n;
        tot_part += Li;
        if (i < b)
            pre_part += Li;
        if (i == lane)
            L_first = Li;
    }
    const int64_t tot = wave_total(tot_part);
    const int64_t pre_b = wave_total(pre_part);
    int64_t P;
    if (fixed_P > 0) {
        P = fixed_P;
    } else {
        P = (tot + nwg - 1) / nwg;
        P = ((P + kTile - 1) / kTile) * kTile;
        if (P < kTile)
            P = kTile;
    }

    const int h = item / NDC, dc = item % NDC;
    const int sl = lane / NQ, qd = lane % NQ;
    const int d0 = dc * DCH + qd * 4;
    __bf16 *dst = out + ((int64_t)b * H + h) * D + d0;
    const int L = b < 64 ? __builtin_amdgcn_readlane(L_first, b) : seq_span(seqlens[b], Tmax, append, window).n;
    if (L == 0) {
        if (sl == 0)
            *reinterpret_cast<u32x2_t *>(dst) = (u32x2_t){0, 0};
        return;
    }
    const int64_t k_first = pre_b / P;
    const int64_t k_last = (pre_b + L - 1) / P;
    if (k_first == k_last)
        return;  // written whole by the decode kernel
    const int nslots = (int)(k_last - k_first + 1);

    float m = -INFINITY, den = 0.f;
    f32x4_t num = {0.f, 0.f, 0.f, 0.f};
    constexpr int U = 4;  // slots per lane per round, loads issued together
    for (int j0 = sl; j0 < nslots; j0 += NS * U) {
        float x[U];
        f32x4_t pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(j0 + NS * u, nslots - 1);
            const int64_t idx = (k_first + j + b) * H + h;  // slot of piece k_first + j
            x[u] = lse[idx];
            pv[u] = *reinterpret_cast<const f32x4_t *>(part + idx * D + d0);
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
    // combine the slot lanes of each d-quad (lanes qd, qd + NQ, ...)
    float M = m;
#pragma unroll
    for (int s = 32; s >= NQ; s >>= 1)
        M = wave_max_xor(M, s);
    const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
    den *= f;
    num *= f;
#pragma unroll
    for (int s = 32; s >= NQ; s >>= 1) {
        den += __shfl_xor(den, s, 64);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            num[e] += __shfl_xor(num[e], s, 64);
    }
    if (sl == 0) {
        const float inv = 1.f / den;
        u32x2_t u = {pack2<T>(num[0] * inv, num[1] * inv), pack2<T>(num[2] * inv, num[3] * inv)};
        *reinterpret_cast<u32x2_t *>(dst) = u;
    }
}

template <typename T, int D, int NQ>
hipError_t launch_merge(const DecodePlan &p, const DecodeArgs &a)
{
    constexpr int NDC = D / (4 * NQ);
    dim3 grid((unsigned)((a.H * NDC + 3) / 4), (unsigned)a.B);
    decode_merge_kernel<T, D, NQ><<<grid, 256, 0, a.stream>>>(a.seqlens, a.B, a.H, a.Tmax, a.knew != nullptr,
                                                          a.window, p.nwg, p.fixed_P, a.part, a.lse,
                                                          static_cast<__bf16 *>(a.out));
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_merge_d(const DecodePlan &p, const DecodeArgs &a)
{
    switch (p.merge_nq) {
    case 1: return launch_merge<T, D, 1>(p, a);
    case 2: return launch_merge<T, D, 2>(p, a);
    case 4: return launch_merge<T, D, 4>(p, a);
    case 8: return launch_merge<T, D, 8>(p, a);
    case 16: return launch_merge<T, D, 16>(p, a);
    default: return launch_merge<T, D, (D >= 128 ? 32 : 16)>(p, a);
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
    float m = -INFINITY, l = 0.f;
    for (int t = 0; t < L; ++t) {
        const int64_t off = (((int64_t)b * Tmax + sp.lo + t) * G + g) * D;
        const float *kp = (t == t_new) ? knew + new_off : kc + off;
        const float *vp = (t == t_new) ? vnew + new_off : vc + off;
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j)
            dot += qv[j] * kp[lane + 64 * j];
        const float s = wave_sum(dot) * scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int j = 0; j < J; ++j)
            acc[j] = acc[j] * alpha + p * vp[lane + 64 * j];
        m = m_new;
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
        out[row * D + lane + 64 * j] = L > 0 ? acc[j] / l : 0.f;
    if (t_new >= 0 && h % r == 0) {  // the group's first head stores the appended token
        const int64_t off = (((int64_t)b * Tmax + sp.lo + t_new) * G + g) * D;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            kc[off + lane + 64 * j] = knew[new_off + lane + 64 * j];
            vc[off + lane + 64 * j] = vnew[new_off + lane + 64 * j];
        }
    }
}

template <int D, int NT, int WAVES, int GB>
const void *split_symbol()
{
    return reinterpret_cast<const void *>(&decode_split_kernel<__bf16, D, NT, WAVES, GB, false>);
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
            p.nwg, p.fixed_P, static_cast<__bf16 *>(a.out), a.part, a.lse);
    else
        decode_split_kernel<T, D, NT, WAVES, GB, false><<<grid, WAVES * 64, 0, a.stream>>>(
            q, kc, vc, kn, vn, a.seqlens, a.B, a.H, a.G, a.Tmax, a.window, p.r, p.head_tiles, a.scale * kLog2e,
            p.nwg, p.fixed_P, static_cast<__bf16 *>(a.out), a.part, a.lse);
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

hipError_t decode_blocks_per_cu(const DecodePlan &p, int D, int *blocks)
{
    return with_variant(p, D, [&]<int DD, int NTT, int WW, int GG>() {
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, split_symbol<DD, NTT, WW, GG>(), WW * 64, 0);
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
    if (dtype == GQA_FP16)
        return with_variant(p, a.D, [&]<int DD, int NTT, int WW, int GG>() {
            return launch_split<_Float16, DD, NTT, WW, GG>(p, a);
        });
    return with_variant(p, a.D, [&]<int DD, int NTT, int WW, int GG>() {
        return launch_split<__bf16, DD, NTT, WW, GG>(p, a);
    });
}

}  // namespace gqa
