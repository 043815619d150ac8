// decode.hip -- GQA decode kernels for gfx950.
//
// Computes, for every sequence b and query head h of group g = h / r,
//   out[b,h,:] = sum_{t < L_b} softmax_t(scale * q[b,h,:] . K[b,t,g,:]) V[b,t,g,:]
// ("Grouped-Query Attention" (llm-arch-kb): section 1 Premise, every cached
// entry is read at a decode step; section 2 Derivation, The grouping; section
// 3 sketch, scaled scores, softmax over keys, times v).
//
// bf16 kernel design (memory-bound: every K/V byte is read exactly once):
//  * Workgroup = (split of the sequence, key/value group g, sequence b); its
//    waves walk 32-position tiles of the split round-robin and each wave keeps
//    its own online-softmax state; the waves merge through LDS at the end.
//  * All r = H/G query heads of the group share every K/V tile: the heads are
//    the N dimension of 16x16x32 bf16 MFMAs, so one read of a tile serves the
//    whole group.
//  * Scores: S^T[token, head] = K_tile . q^T. K goes from HBM straight into
//    registers in the MFMA A layout (lane = token row, 16-byte chunk of d_h),
//    q sits in registers as the B operand for the whole kernel.
//  * The C layout of S^T (lane holds 4 tokens of one head) is already the B
//    operand layout of P^T for O^T = V^T P^T, with tokens as the contraction
//    index, so P never leaves registers.
//  * V is loaded with fully coalesced 16-byte rows, written to a per-wave LDS
//    tile, and read back with ds_read_b64_tr_b16, which delivers 4 consecutive
//    tokens of one d column per lane: the A operand of V^T.
//  * Softmax statistics are kept in base 2 (scores pre-multiplied by
//    scale*log2(e)); row maxima use two cross-lane exchanges per tile.
//  * A sequence longer than one split is spread over several workgroups; each
//    writes a normalised partial row and its log-sum-exp, and the last
//    workgroup to arrive for a (sequence, group, head tile) merges them, all
//    in one launch.
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

constexpr int kTile = 32;  // positions per wave iteration

template <int D, int NT, int WAVES>
struct DecodeCfg {
    static constexpr int KS = D / 32;          // MFMA k-steps over d_h
    static constexpr int DT = D / 16;          // 16-wide d tiles of the output
    static constexpr int CH = D / 8;           // 16-byte chunks per row
    static constexpr int VROWS = 64 / CH;      // V rows per coalesced load
    static constexpr int VLOADS = kTile / VROWS;
    static constexpr int LDS_STRIDE = D + 16;  // padded row (elements): 4 rows cover all banks
    static constexpr int HEADS = 16 * NT;
    static constexpr int V_LDS_ELEMS = WAVES * kTile * LDS_STRIDE;
    // merge area (floats) aliases the V tiles after the main loop
    static constexpr int RED_FLOATS = HEADS * D + 2 * WAVES * HEADS;
    static constexpr int LDS_BYTES = (V_LDS_ELEMS * 2 > RED_FLOATS * 4) ? V_LDS_ELEMS * 2 : RED_FLOATS * 4;
};

__device__ __forceinline__ u32x4_t load16(const __bf16 *p)
{
    return *reinterpret_cast<const u32x4_t *>(p);
}

template <int D, int NT, int WAVES>
__global__ void __launch_bounds__(WAVES * 64)
decode_bf16_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ kc, const __bf16 *__restrict__ vc,
                   const int32_t *__restrict__ seqlens, int H, int G, int Tmax, int r, int head_tiles,
                   float scale_log2, int chunk, int splits, __bf16 *__restrict__ out,
                   float *__restrict__ part, float *__restrict__ lse, int *__restrict__ counters)
{
    using C = DecodeCfg<D, NT, WAVES>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_BYTES];
    __shared__ int s_last;

    const int split = blockIdx.x;
    const int g = blockIdx.y / head_tiles;
    const int ht = blockIdx.y % head_tiles;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kb = lane >> 4;

    const int L = clamp_len(seqlens[b], Tmax);
    const int t_begin = split * chunk;
    const int n_active = (L + chunk - 1) / chunk;
    const int h0 = g * r + ht * C::HEADS;                  // first query head of this tile
    const int nheads = min(C::HEADS, r - ht * C::HEADS);   // valid heads in this tile
    const int64_t row0 = (int64_t)b * H + h0;              // first output row

    if (t_begin >= L) {
        if (split == 0) {  // empty sequence: zero rows
            for (int i = tid; i < nheads * C::CH; i += WAVES * 64) {
                const int hh = i / C::CH, c = i % C::CH;
                *reinterpret_cast<u32x4_t *>(out + (row0 + hh) * D + c * 8) = (u32x4_t){0, 0, 0, 0};
            }
        }
        return;
    }
    const int t_end = min(t_begin + chunk, L);

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
    const __bf16 *kbase = kc + ((int64_t)b * Tmax * G + g) * D;
    const __bf16 *vbase = vc + ((int64_t)b * Tmax * G + g) * D;
    __bf16 *vl = reinterpret_cast<__bf16 *>(smem) + wave * kTile * C::LDS_STRIDE;

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

    u32x4_t kcur[2][C::KS], vcur[C::VLOADS];
    auto load_tile = [&](int t0, u32x4_t (&kr)[2][C::KS], u32x4_t (&vr)[C::VLOADS]) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int t = t0 + mt * 16 + col;
#pragma unroll
            for (int s = 0; s < C::KS; ++s) {
                u32x4_t v = {0, 0, 0, 0};
                if (t < t_end)
                    v = load16(kbase + t * tok_stride + (s * 4 + kb) * 8);
                kr[mt][s] = v;
            }
        }
#pragma unroll
        for (int i = 0; i < C::VLOADS; ++i) {
            const int t = t0 + i * C::VROWS + lane / C::CH;
            u32x4_t v = {0, 0, 0, 0};
            if (t < t_end)
                v = load16(vbase + t * tok_stride + (lane % C::CH) * 8);
            vr[i] = v;
        }
    };

    int t0 = t_begin + wave * kTile;
    if (t0 < t_end)
        load_tile(t0, kcur, vcur);
    while (t0 < t_end) {
        const int tn = t0 + WAVES * kTile;
        u32x4_t knext[2][C::KS], vnext[C::VLOADS];
        if (tn < t_end)
            load_tile(tn, knext, vnext);

        // V tile into this wave's LDS rows (natural [token][d] order).
        compiler_fence();
#pragma unroll
        for (int i = 0; i < C::VLOADS; ++i)
            *reinterpret_cast<u32x4_t *>(vl + (i * C::VROWS + lane / C::CH) * C::LDS_STRIDE + (lane % C::CH) * 8) =
                vcur[i];
        compiler_fence();

        // S^T = K q^T for two 16-token row tiles.
        f32x4_t st[2][NT];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < C::KS; ++s)
                    c = mfma16x16x32(__builtin_bit_cast(bf16x8_t, kcur[mt][s]), qf[nt][s], c);
                st[mt][nt] = c;
            }

        // Online softmax (base 2). Lane holds tokens t0 + 16*mt + 4*kb + i of head column col.
        bf16x8_t pf[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = t0 + mt * 16 + kb * 4 + i;
                    const float x = (t < t_end) ? st[mt][nt][i] * scale_log2 : -INFINITY;
                    st[mt][nt][i] = x;
                    mx = fmaxf(mx, x);
                }
            mx = wave_max_xor(mx, 16);
            mx = wave_max_xor(mx, 32);
            const float m_new = fmaxf(m_run[nt], mx);
            const float alpha = fast_exp2(m_run[nt] - m_new);
            m_run[nt] = m_new;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[mt][nt][i] = fast_exp2(st[mt][nt][i] - m_new);
            pf[nt] = pack_bf16x8(st[0][nt], st[1][nt]);
            // The denominator sums the same bf16-rounded weights that enter
            // the P.V product, so the output is a convex combination of V rows.
            const u32x4_t pu = __builtin_bit_cast(u32x4_t, pf[nt]);
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                psum += bf16_bits_to_f32(pu[j] & 0xffffu) + bf16_bits_to_f32(pu[j] >> 16);
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
                acc[nt][dt] = mfma16x16x32(vf, pf[nt], acc[nt][dt]);
        }

        if (tn < t_end) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int s = 0; s < C::KS; ++s)
                    kcur[mt][s] = knext[mt][s];
#pragma unroll
            for (int i = 0; i < C::VLOADS; ++i)
                vcur[i] = vnext[i];
        }
        t0 = tn;
    }

    // ---- merge the waves of this workgroup -------------------------------
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        l_run[nt] += __shfl_xor(l_run[nt], 16, 64);
        l_run[nt] += __shfl_xor(l_run[nt], 32, 64);
    }
    __syncthreads();  // every wave is done with its V tile
    float *red = reinterpret_cast<float *>(smem);          // [HEADS][D]
    float *wm = red + C::HEADS * D;                         // [WAVES][HEADS]
    float *wl = wm + WAVES * C::HEADS;                      // [WAVES][HEADS]
    if (kb == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            wm[wave * C::HEADS + nt * 16 + col] = m_run[nt];
            wl[wave * C::HEADS + nt * 16 + col] = l_run[nt];
        }
    }
    __syncthreads();
    // Wave w adds its rescaled accumulator after waves 0..w-1 (fixed order,
    // so repeated launches give identical bits).
    float f[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int hh = nt * 16 + col;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w)
            M = fmaxf(M, wm[w * C::HEADS + hh]);
        f[nt] = (m_run[nt] == -INFINITY) ? 0.f : fast_exp2(m_run[nt] - M);
    }
    for (int w = 0; w < WAVES; ++w) {
        if (wave == w) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int hh = nt * 16 + col;
                if (hh < nheads) {
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float *dst = &red[hh * D + dt * 16 + kb * 4 + i];
                            const float x = acc[nt][dt][i] * f[nt];
                            *dst = (w == 0) ? x : *dst + x;
                        }
                }
            }
        }
        __syncthreads();
    }

    // Per-head totals of this workgroup: max M and sum l scaled to M.
    auto head_stats = [&](int hh, float &M, float &Ls) {
        M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w)
            M = fmaxf(M, wm[w * C::HEADS + hh]);
        Ls = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float mw = wm[w * C::HEADS + hh];
            if (mw != -INFINITY)
                Ls += wl[w * C::HEADS + hh] * fast_exp2(mw - M);
        }
    };

    if (n_active == 1) {  // the whole sequence was in this workgroup
        for (int i = tid; i < nheads * C::CH; i += WAVES * 64) {
            const int hh = i / C::CH, c = i % C::CH;
            float M, Ls;
            head_stats(hh, M, Ls);
            const float inv = 1.f / Ls;
            const float *src = red + hh * D + c * 8;
            u32x4_t o;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = pack_bf16x2(src[2 * j] * inv, src[2 * j + 1] * inv);
            *reinterpret_cast<u32x4_t *>(out + (row0 + hh) * D + c * 8) = o;
        }
        return;
    }

    // Several workgroups share this sequence: write a normalised partial row
    // and its base-2 log-sum-exp.
    for (int i = tid; i < nheads * (D / 4); i += WAVES * 64) {
        const int hh = i / (D / 4), c = i % (D / 4);
        float M, Ls;
        head_stats(hh, M, Ls);
        const float inv = 1.f / Ls;
        const float *src = red + hh * D + c * 4;
        f32x4_t o = {src[0] * inv, src[1] * inv, src[2] * inv, src[3] * inv};
        *reinterpret_cast<f32x4_t *>(part + ((row0 + hh) * splits + split) * D + c * 4) = o;
        if (c == 0)
            lse[(row0 + hh) * splits + split] = M + fast_log2(Ls);
    }
    __threadfence();
    __syncthreads();
    const int pair = (b * G + g) * head_tiles + ht;
    if (tid == 0) {
        const int prev = atomicAdd(&counters[pair], 1);
        s_last = (prev == n_active - 1);
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();

    // Last arrival: merge the n_active partial rows of every head.
    for (int i = tid; i < nheads * C::CH; i += WAVES * 64) {
        const int hh = i / C::CH, c = i % C::CH;
        const int64_t row = row0 + hh;
        const float *lrow = lse + row * splits;
        float M = -INFINITY;
        for (int s = 0; s < n_active; ++s)
            M = fmaxf(M, lrow[s]);
        float den = 0.f;
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < n_active; ++s) {
            const float w = fast_exp2(lrow[s] - M);
            const f32x4_t *src = reinterpret_cast<const f32x4_t *>(part + (row * splits + s) * D + c * 8);
            a0 += w * src[0];
            a1 += w * src[1];
            den += w;
        }
        const float inv = 1.f / den;
        u32x4_t o;
        o[0] = pack_bf16x2(a0[0] * inv, a0[1] * inv);
        o[1] = pack_bf16x2(a0[2] * inv, a0[3] * inv);
        o[2] = pack_bf16x2(a1[0] * inv, a1[1] * inv);
        o[3] = pack_bf16x2(a1[2] * inv, a1[3] * inv);
        *reinterpret_cast<u32x4_t *>(out + row * D + c * 8) = o;
    }
    if (tid == 0)
        atomicExch(&counters[pair], 0);  // ready for the next launch
}

// fp32 debug path: one wavefront per (sequence, head); lanes split d_h and the
// wave walks the cache one position at a time with an online softmax.
template <int D>
__global__ void __launch_bounds__(64)
decode_f32_kernel(const float *__restrict__ q, const float *__restrict__ kc, const float *__restrict__ vc,
                  const int32_t *__restrict__ seqlens, int H, int G, int Tmax, int r, float scale,
                  float *__restrict__ out)
{
    constexpr int J = D / 64;
    const int64_t row = blockIdx.x;
    const int b = (int)(row / H), h = (int)(row % H);
    const int g = h / r;
    const int lane = threadIdx.x;
    const int L = clamp_len(seqlens[b], Tmax);
    float qv[J], acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        qv[j] = q[row * D + lane + 64 * j];
        acc[j] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int t = 0; t < L; ++t) {
        const float *kp = kc + (((int64_t)b * Tmax + t) * G + g) * D;
        const float *vp = vc + (((int64_t)b * Tmax + t) * G + g) * D;
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
}

template <int D, int NT, int WAVES>
hipError_t launch_bf16(const DecodePlan &p, const DecodeArgs &a)
{
    dim3 grid(p.splits, a.G * p.head_tiles, a.B);
    decode_bf16_kernel<D, NT, WAVES><<<grid, WAVES * 64, 0, a.stream>>>(
        static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), static_cast<const __bf16 *>(a.v),
        a.seqlens, a.H, a.G, a.Tmax, p.r, p.head_tiles, a.scale * kLog2e, p.chunk, p.splits,
        static_cast<__bf16 *>(a.out), a.part, a.lse, a.counters);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(const DecodePlan &p, const DecodeArgs &a)
{
    switch (p.nt) {
    case 1: return launch_bf16<D, 1, 4>(p, a);
    case 2: return launch_bf16<D, 2, 4>(p, a);
    default: return launch_bf16<D, 4, 4>(p, a);
    }
}

}  // namespace

hipError_t launch_decode(const DecodePlan &p, const DecodeArgs &a, gqa_dtype dtype)
{
    if (dtype == GQA_FP32) {
        dim3 grid((unsigned)((int64_t)a.B * a.H));
        if (a.D == 64)
            decode_f32_kernel<64><<<grid, 64, 0, a.stream>>>(
                static_cast<const float *>(a.q), static_cast<const float *>(a.k), static_cast<const float *>(a.v),
                a.seqlens, a.H, a.G, a.Tmax, p.r, a.scale, static_cast<float *>(a.out));
        else
            decode_f32_kernel<128><<<grid, 64, 0, a.stream>>>(
                static_cast<const float *>(a.q), static_cast<const float *>(a.k), static_cast<const float *>(a.v),
                a.seqlens, a.H, a.G, a.Tmax, p.r, a.scale, static_cast<float *>(a.out));
        return hipGetLastError();
    }
    return a.D == 64 ? launch_bf16_d<64>(p, a) : launch_bf16_d<128>(p, a);
}

}  // namespace gqa
