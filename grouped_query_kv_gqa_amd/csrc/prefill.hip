// prefill.hip -- GQA prefill (every position of a sequence is a query).
//
// out[b,t,h,:] = sum_{s in keys(t)} softmax_s(q[b,t,h,:] . k[b,s,g,:] / sqrt(d_h)) v[b,s,g,:]
// with g = h / r and keys(t) = [0, t] when causal, [0, T) otherwise
// ("Grouped-Query Attention" (llm-arch-kb), section 3 Reference
// implementation: broadcast of each key/value head to its H/G query heads,
// scores over sqrt(d_h), causal mask, softmax over keys, times v).
//
// bf16 MFMA kernel (flash-attention style, one pass over keys with an online
// softmax; the score matrix never leaves registers):
//  * Workgroup = (query tile, key/value group g, sequence b). Its 128 query
//    rows are (token, head) pairs: QT = 128 / r consecutive tokens times the r
//    heads of group g, so one K/V tile in LDS serves all heads of the group
//    (the broadcast of the sketch costs no extra memory traffic).
//  * 4 waves x 32 rows. Scores are computed transposed, S^T = K . Q^T, with
//    32x32x16 bf16 MFMAs (keys in M, query rows in N): the result layout (a
//    lane holds 16 keys of one row) is directly the B operand P^T of
//    O^T = V^T . P^T, so P stays in registers.
//  * K/V tiles of 64 positions are double-buffered in LDS and loaded straight
//    from global memory into LDS (global_load_lds_dwordx4, no staging
//    registers); the next tile lands while the current one is used. Rows are
//    unpadded with XOR-swizzled 16-byte chunks so that the 16-byte K reads and
//    the V^T transposing reads (ds_read_b64_tr_b16) avoid bank conflicts.
//  * Causal: a query tile only visits key tiles up to its last token; the
//    heaviest tiles are launched first.
//  * Softmax in base 2 against a lazily moved per-row reference (rescaling
//    only when a row maximum grows by more than 2^8); masking only on the
//    tiles that cross the causal diagonal or the sequence end.
//
// Row kernel (fp32 path, and groups of more than 128 query heads): one
// wavefront per (b, t, h) row, lanes split d_h, online softmax over the keys
// one position at a time, fp32 arithmetic.
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T *p);
template <>
__device__ __forceinline__ float ld<float>(const float *p)
{
    return *p;
}
template <>
__device__ __forceinline__ float ld<__bf16>(const __bf16 *p)
{
    return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(p));
}

template <typename T>
__device__ __forceinline__ void st(T *p, float x);
template <>
__device__ __forceinline__ void st<float>(float *p, float x)
{
    *p = x;
}
template <>
__device__ __forceinline__ void st<__bf16>(__bf16 *p, float x)
{
    *reinterpret_cast<uint16_t *>(p) = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}

template <typename T, int D>
__global__ void __launch_bounds__(64)
prefill_row_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, int T_, int H,
                   int G, int causal, float scale, T *__restrict__ out)
{
    constexpr int J = D / 64;
    const int64_t row = blockIdx.x;  // ((b * T) + t) * H + h
    const int h = (int)(row % H);
    const int64_t bt = row / H;
    const int t = (int)(bt % T_);
    const int64_t b = bt / T_;
    const int r = H / G;
    const int g = h / r;
    const int lane = threadIdx.x;
    const int nkeys = causal ? t + 1 : T_;
    float qv[J], acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        qv[j] = ld(q + row * D + lane + 64 * j);
        acc[j] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int s = 0; s < nkeys; ++s) {
        const int64_t off = ((b * T_ + s) * G + g) * D;
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j)
            dot += qv[j] * ld(k + off + lane + 64 * j);
        const float sc = wave_sum(dot) * scale;
        const float m_new = fmaxf(m, sc);
        const float alpha = expf(m - m_new);
        const float p = expf(sc - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int j = 0; j < J; ++j)
            acc[j] = acc[j] * alpha + p * ld(v + off + lane + 64 * j);
        m = m_new;
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
        st(out + row * D + lane + 64 * j, acc[j] / l);
}

template <typename T>
hipError_t launch_rows(const PrefillArgs &a)
{
    const int64_t rows = (int64_t)a.B * a.T * a.H;
    const float scale = 1.0f / sqrtf((float)a.D);
    if (a.D == 64)
        prefill_row_kernel<T, 64><<<dim3((unsigned)rows), 64, 0, a.stream>>>(
            static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v), a.T, a.H, a.G,
            a.causal, scale, static_cast<T *>(a.out));
    else
        prefill_row_kernel<T, 128><<<dim3((unsigned)rows), 64, 0, a.stream>>>(
            static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v), a.T, a.H, a.G,
            a.causal, scale, static_cast<T *>(a.out));
    return hipGetLastError();
}

constexpr int kPfBN = 64;  // key/value positions per tile
#ifndef GQA_PREFILL_NTW
#define GQA_PREFILL_NTW 1
#endif
constexpr int kPfNTW = GQA_PREFILL_NTW;  // 32-row column tiles per wave

template <int D, int NTW>
struct PfCfg {
    static constexpr int ROWS = 4 * 32 * NTW;           // query rows per workgroup (4 waves)
    static constexpr int KS = D / 16;                   // QK k-steps over d_h
    static constexpr int DT = D / 32;                   // 32-wide d tiles of O^T
    static constexpr int CH = D / 8;                    // 16-byte chunks per row
    static constexpr int WAVE_ROWS = 64 / CH;           // rows one wave load instruction fills
    static constexpr int LOADS = kPfBN / (4 * WAVE_ROWS); // load instructions per tensor per wave
    static constexpr int TILE_ELEMS = kPfBN * D;        // unpadded rows, chunks swizzled
};

// LDS tile layout: rows of d_h elements without padding; the 16-byte chunk c
// of row r sits at chunk slot c ^ kswz(r) (K) or c ^ vswz(r) (V). K is read
// 16 rows at a time at one chunk (b128 reads): r mod 16 spreads them over 16
// slots. V is read by the transposing loads 4 rows x 2 chunks at a time:
// 2*(r mod 4) spreads those over 8 slots.
template <int D>
struct PfSwz {
    static __device__ __forceinline__ int k(int r) { return r & (D / 8 - 1); }
    static __device__ __forceinline__ int v(int r) { return (r & 3) << 1; }
};

__device__ __forceinline__ u32x4_t ld16(const __bf16 *p)
{
    return *reinterpret_cast<const u32x4_t *>(p);
}

// NTW = 32-row MFMA column tiles per wave: every K/V fragment read from LDS
// feeds NTW independent MFMAs. With NTW = 2 a wave holds 64 query rows (its
// accumulators live in AGPRs) and one 4-wave workgroup fills a compute unit.
template <int D, int NTW>
__global__ void __launch_bounds__(256, NTW == 1 ? 2 : 1)
prefill_bf16_kernel(const __bf16 *__restrict__ q, const __bf16 *kp, const __bf16 *vp, int T, int H, int G, int r,
                    int QT, int causal, float scale_log2, __bf16 *__restrict__ out)
{
    using C = PfCfg<D, NTW>;
    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][C::TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[2][C::TILE_ELEMS];
    using SW = PfSwz<D>;

    const int qt = gridDim.x - 1 - blockIdx.x;  // heaviest causal tiles first
    const int g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int t0 = qt * QT;

    // This lane's query rows: column n of the wave's NTW S^T column tiles.
    int tq[NTW];
    bool row_ok[NTW];
    int64_t qrow[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int rho = (wave * NTW + nt) * 32 + n;
        tq[nt] = t0 + rho / r;
        row_ok[nt] = rho < QT * r && tq[nt] < T;
        qrow[nt] = ((int64_t)b * T + min(tq[nt], T - 1)) * H + g * r + rho % r;
    }
    const int t_row_min = t0 + (wave * NTW * 32) / r;  // first query token of this wave

    // Q^T as the B operand: lane holds q[row][16*ks + 8*h .. +7].
    bf16x8_t qf[NTW][C::KS];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            u32x4_t x = {0, 0, 0, 0};
            if (row_ok[nt])
                x = ld16(q + qrow[nt] * D + ks * 16 + h * 8);
            qf[nt][ks] = __builtin_bit_cast(bf16x8_t, x);
        }

    const int t_hi = min(T, t0 + QT);
    const int kv_end = causal ? t_hi : T;
    const int ntiles = (kv_end + kPfBN - 1) / kPfBN;

    // Tile loads go straight from global memory into LDS
    // (global_load_lds_dwordx4): lane i of a wave instruction fills the
    // 16-byte LDS slot base + 16*i, i.e. row WAVE_ROWS*instr + i/CH, slot
    // i%CH, so it fetches the global chunk that the swizzle puts in that slot.
    // Rows past the sequence end are clamped to its last row: their scores
    // are masked to -inf, so they meet p = 0 with finite values.
    const int srow = lane / C::CH, sslot = lane % C::CH;
    auto tile_load = [&](int buf, int tile) {
#pragma unroll
        for (int u = 0; u < C::LOADS; ++u) {
            const int rl = (u * 4 + wave) * C::WAVE_ROWS + srow;  // tile row of this lane
            const int t = min(tile * kPfBN + rl, T - 1);
            const int64_t goff = (((int64_t)b * T + t) * G + g) * D;
            const int lbase = (u * 4 + wave) * C::WAVE_ROWS * D;   // wave-uniform LDS base
            __builtin_amdgcn_global_load_lds(
                (__attribute__((address_space(1))) void *)(kp + goff + (sslot ^ SW::k(rl)) * 8),
                (__attribute__((address_space(3))) void *)&Ks[buf][lbase], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (__attribute__((address_space(1))) void *)(vp + goff + (sslot ^ SW::v(rl)) * 8),
                (__attribute__((address_space(3))) void *)&Vs[buf][lbase], 16, 0, 0);
        }
    };

    f32x16_t acc[NTW][C::DT];
    float m_run[NTW], l_run[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
            acc[nt][dt] = (f32x16_t){};
    }

    tile_load(0, 0);
    for (int j = 0; j < ntiles; ++j) {
        const int cur = j & 1;
        wait_vector_memory();  // this wave's loads of tile j have landed in LDS
        __syncthreads();       // everyone's have; every wave is done with tile j-1
        if (j + 1 < ntiles)
            tile_load(cur ^ 1, j + 1);  // lands while tile j is used

        // S^T = K Q^T: two 32-key M tiles x NTW row tiles. Each K fragment
        // (read from LDS one k-step ahead) feeds NTW independent MFMAs, and
        // the M tiles alternate so consecutive MFMAs never share an
        // accumulator.
        f32x16_t st[NTW][2];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
            st[nt][0] = st[nt][1] = (f32x16_t){};
        {
            // lane (n, h) reads chunk 2*ks + h of rows n and 32 + n
            const __bf16 *krow0 = &Ks[cur][n * D];
            const __bf16 *krow1 = krow0 + 32 * D;
            const int sw = SW::k(n);  // rows n and n + 32 share the swizzle
            auto kfrag = [&](const __bf16 *row, int ks) {
                return __builtin_bit_cast(bf16x8_t, ld16(row + ((2 * ks + h) ^ sw) * 8));
            };
            bf16x8_t ka0 = kfrag(krow0, 0);
            bf16x8_t ka1 = kfrag(krow1, 0);
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                bf16x8_t kb0 = ka0, kb1 = ka1;
                if (ks + 1 < C::KS) {
                    kb0 = kfrag(krow0, ks + 1);
                    kb1 = kfrag(krow1, ks + 1);
                }
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    st[nt][0] = mfma32x32x16(ka0, qf[nt][ks], st[nt][0]);
                    st[nt][1] = mfma32x32x16(ka1, qf[nt][ks], st[nt][1]);
                }
                ka0 = kb0;
                ka1 = kb1;
            }
        }

        // Online softmax in base 2 with a lazily moved reference m_run (in
        // scaled units): p = 2^(s*c - m_run) with c = scale*log2(e). The
        // reference only moves, rescaling O and l, when a row's maximum
        // exceeds it by more than kLazy, so p <= 2^kLazy; softmax is
        // unchanged by the choice of reference. Register v of tile mt holds
        // key j*64 + 32*mt + 8*(v/4) + 4*h + v%4. Only tiles that cross this
        // wave's causal diagonal or the sequence end need masking.
        constexpr float kLazy = 8.f;
        const int tile_last = j * kPfBN + kPfBN - 1;
        const bool need_mask = causal ? (tile_last > t_row_min) : (tile_last >= T);
        if (need_mask) {
            const int tk0 = j * kPfBN + 4 * h;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const int key_lim = causal ? tq[nt] : T - 1;  // last admissible key
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int tk = tk0 + 32 * mt + 8 * (v >> 2) + (v & 3);
                        st[nt][mt][v] = (tk <= key_lim) ? st[nt][mt][v] : -INFINITY;
                    }
            }
        }
        bool move[NTW];
        float m_old[NTW];
        bool any_move = false;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int v = 0; v < 16; v += 2)
                    mx = fmaxf(mx, fmaxf(st[nt][mt][v], st[nt][mt][v + 1]));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
            move[nt] = mx > m_run[nt] + kLazy;
            m_old[nt] = m_run[nt];
            m_run[nt] = move[nt] ? mx : m_run[nt];
            any_move |= move[nt];
        }
        if (__any(any_move)) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const float alpha = (m_old[nt] == -INFINITY) ? 0.f : fast_exp2(m_old[nt] - m_run[nt]);
                l_run[nt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
                    acc[nt][dt] *= alpha;
            }
        }
        bf16x8_t pf[NTW][4];  // P^T for k-step (mt, qh) = 2*mt + qh
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const float m_use = (m_run[nt] == -INFINITY) ? 0.f : m_run[nt];
            float psum = 0.f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int qh = 0; qh < 2; ++qh) {
                    f32x4_t a, c;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        a[i] = fast_exp2(fmaf(st[nt][mt][8 * qh + i], scale_log2, -m_use));
                        c[i] = fast_exp2(fmaf(st[nt][mt][8 * qh + 4 + i], scale_log2, -m_use));
                        psum += a[i] + c[i];
                    }
                    pf[nt][2 * mt + qh] = pack_bf16x8(a, c);
                }
            l_run[nt] += psum;
        }

        // O^T += V^T P^T: k-step (mt, qh) covers keys 32*mt + 16*qh +
        // {4h..4h+3, 8+4h..8+4h+3}. Each V^T fragment feeds NTW MFMAs with
        // different accumulators.
        const int i16 = lane & 15, nh = n >> 4;
        // lane reads row 32*mt + 16*qh + 4*h + i16/4 (and 8 rows on), columns
        // dt*32 + 16*nh + 4*(i16%4) .. +3: chunk 4*dt + 2*nh + (i16%4)/2, half (i16%2)
        auto vfrag = [&](int kstep, int dt) {
            const int mt = kstep >> 1, qh = kstep & 1;
            const int row = 32 * mt + 16 * qh + 4 * h + (i16 >> 2);
            const int chunk = 4 * dt + 2 * nh + ((i16 & 3) >> 1);
            const int half = (i16 & 1) * 4;
            const __bf16 *p0 = &Vs[cur][row * D + ((chunk ^ SW::v(row)) * 8) + half];
            const __bf16 *p1 = &Vs[cur][(row + 8) * D + ((chunk ^ SW::v(row + 8)) * 8) + half];
            const bf16x4_t lo = lds_read_tr16(p0);
            const bf16x4_t hi = lds_read_tr16(p1);
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep)
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                const bf16x8_t va = vfrag(kstep, dt);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    acc[nt][dt] = mfma32x32x16(va, pf[nt][kstep], acc[nt][dt]);
            }

    }

    // Epilogue: lane holds O^T[dt*32 + 8*m0 + 4*h + m1][row]; 4 consecutive d per (dt, m0).
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const float lsum = l_run[nt] + __shfl_xor(l_run[nt], 32, 64);
        if (!row_ok[nt])
            continue;
        const float inv = 1.f / lsum;
        __bf16 *dst = out + qrow[nt] * D + 4 * h;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int m0 = 0; m0 < 4; ++m0) {
                u32x2_t u = {pack_bf16x2(acc[nt][dt][4 * m0] * inv, acc[nt][dt][4 * m0 + 1] * inv),
                             pack_bf16x2(acc[nt][dt][4 * m0 + 2] * inv, acc[nt][dt][4 * m0 + 3] * inv)};
                *reinterpret_cast<u32x2_t *>(dst + dt * 32 + 8 * m0) = u;
            }
    }
}

template <int D, int NTW>
hipError_t launch_mfma(const PrefillArgs &a)
{
    const int r = a.H / a.G;
    const int QT = PfCfg<D, NTW>::ROWS / r;
    const int nqt = (a.T + QT - 1) / QT;
    const float scale_log2 = kLog2e / sqrtf((float)D);
    prefill_bf16_kernel<D, NTW><<<dim3(nqt, a.G, a.B), 256, 0, a.stream>>>(
        static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), static_cast<const __bf16 *>(a.v), a.T,
        a.H, a.G, r, QT, a.causal, scale_log2, static_cast<__bf16 *>(a.out));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, gqa_dtype dtype)
{
    if (dtype == GQA_FP32)
        return launch_rows<float>(a);
    if (a.H / a.G > PfCfg<128, kPfNTW>::ROWS)
        return launch_rows<__bf16>(a);
    return a.D == 64 ? launch_mfma<64, kPfNTW>(a) : launch_mfma<128, kPfNTW>(a);
}

}  // namespace gqa
