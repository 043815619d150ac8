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
//  * K/V tiles of 64 positions are double-buffered in LDS: the next tile's
//    global loads are in flight while the current one is used. K fragments
//    are read with 16-byte LDS reads (rows padded by 16 bytes), V^T fragments
//    with ds_read_b64_tr_b16 (rows padded by 32 bytes).
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

constexpr int kPfRows = 128;  // query rows (token, head) per workgroup
constexpr int kPfBN = 64;     // key/value positions per tile

template <int D>
struct PfCfg {
    static constexpr int KS = D / 16;                   // QK k-steps over d_h
    static constexpr int DT = D / 32;                   // 32-wide d tiles of O^T
    static constexpr int KSTRIDE = D + 8;               // K row stride (elements)
    static constexpr int VSTRIDE = D + 16;              // V row stride (elements)
    static constexpr int CH = D / 8;                    // 16-byte chunks per row
    static constexpr int ROWS_PER_LOAD = 256 / CH;      // rows per cooperative load
    static constexpr int LOADS = kPfBN / ROWS_PER_LOAD; // loads per tensor per thread
    static constexpr int K_ELEMS = kPfBN * KSTRIDE;
    static constexpr int V_ELEMS = kPfBN * VSTRIDE;
};

__device__ __forceinline__ u32x4_t ld16(const __bf16 *p)
{
    return *reinterpret_cast<const u32x4_t *>(p);
}

template <int D>
__global__ void __launch_bounds__(256, 2)
prefill_bf16_kernel(const __bf16 *__restrict__ q, const __bf16 *kp, const __bf16 *vp, int T, int H, int G, int r,
                    int QT, int causal, float scale_log2, __bf16 *__restrict__ out)
{
    using C = PfCfg<D>;
    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][C::K_ELEMS];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[2][C::V_ELEMS];

    const int qt = gridDim.x - 1 - blockIdx.x;  // heaviest causal tiles first
    const int g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int t0 = qt * QT;

    // This lane's query row: column n of the wave's S^T tiles.
    const int rho = wave * 32 + n;
    const int tq = t0 + rho / r;
    const int jh = rho % r;
    const bool row_ok = rho < QT * r && tq < T;
    const int t_row_min = t0 + (wave * 32) / r;  // first query token of this wave
    const int64_t qrow = ((int64_t)b * T + min(tq, T - 1)) * H + g * r + jh;

    // Q^T as the B operand: lane holds q[row][16*ks + 8*h .. +7].
    bf16x8_t qf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        u32x4_t x = {0, 0, 0, 0};
        if (row_ok)
            x = ld16(q + qrow * D + ks * 16 + h * 8);
        qf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }

    const int t_hi = min(T, t0 + QT);
    const int kv_end = causal ? t_hi : T;
    const int ntiles = (kv_end + kPfBN - 1) / kPfBN;

    // Cooperative tile loads: thread -> (row tid/CH + ROWS_PER_LOAD*u, chunk tid%CH).
    const int lrow = tid / C::CH, lch = tid % C::CH;
    auto gload = [&](int tile, u32x4_t (&kr)[C::LOADS], u32x4_t (&vr)[C::LOADS]) {
#pragma unroll
        for (int u = 0; u < C::LOADS; ++u) {
            const int t = min(tile * kPfBN + lrow + C::ROWS_PER_LOAD * u, T - 1);
            const int64_t off = (((int64_t)b * T + t) * G + g) * D + lch * 8;
            kr[u] = ld16(kp + off);
            vr[u] = ld16(vp + off);
        }
    };
    auto lstore = [&](int buf, int tile, const u32x4_t (&kr)[C::LOADS], const u32x4_t (&vr)[C::LOADS]) {
#pragma unroll
        for (int u = 0; u < C::LOADS; ++u) {
            const int rl = lrow + C::ROWS_PER_LOAD * u;
            const u32x4_t zero = {0, 0, 0, 0};
            *reinterpret_cast<u32x4_t *>(&Ks[buf][rl * C::KSTRIDE + lch * 8]) = kr[u];
            *reinterpret_cast<u32x4_t *>(&Vs[buf][rl * C::VSTRIDE + lch * 8]) =
                (tile * kPfBN + rl < T) ? vr[u] : zero;
        }
    };

    f32x16_t acc[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
        acc[dt] = (f32x16_t){};
    float m_run = -INFINITY, l_run = 0.f;

    u32x4_t kr[C::LOADS], vr[C::LOADS];
    gload(0, kr, vr);
    lstore(0, 0, kr, vr);
    for (int j = 0; j < ntiles; ++j) {
        const int cur = j & 1;
        const bool more = j + 1 < ntiles;
        if (more)
            gload(j + 1, kr, vr);  // in flight while tile j is used
        __syncthreads();           // tile j visible; every wave is done with tile j-1

        // S^T = K Q^T, two 32-key M tiles.
        f32x16_t st[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            f32x16_t c = {};
            const __bf16 *krow = &Ks[cur][(mt * 32 + n) * C::KSTRIDE + h * 8];
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                c = mfma32x32x16(__builtin_bit_cast(bf16x8_t, ld16(krow + ks * 16)), qf[ks], c);
            st[mt] = c;
        }

        // Online softmax in base 2 with a lazily moved reference m_run (in
        // scaled units): p = 2^(s*c - m_run) with c = scale*log2(e). The
        // reference only moves, rescaling O and l, when a row's maximum
        // exceeds it by more than kLazy, so p <= 2^kLazy; softmax is
        // unchanged by the choice of reference. Register v of tile mt holds
        // key j*64 + 32*mt + 8*(v/4) + 4*h + v%4 of row tq. Only tiles that
        // cross this wave's causal diagonal or the sequence end need masking.
        constexpr float kLazy = 8.f;
        const int tile_last = j * kPfBN + kPfBN - 1;
        const bool need_mask = causal ? (tile_last > t_row_min) : (tile_last >= T);
        if (need_mask) {
            const int tk0 = j * kPfBN + 4 * h;
            const int key_lim = causal ? tq : T - 1;  // last admissible key
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int tk = tk0 + 32 * mt + 8 * (v >> 2) + (v & 3);
                    st[mt][v] = (tk <= key_lim) ? st[mt][v] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; v += 2)
                mx = fmaxf(mx, fmaxf(st[mt][v], st[mt][v + 1]));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
        const bool move = mx > m_run + kLazy;
        if (__any(move)) {
            const float m_new = move ? mx : m_run;
            const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
                acc[dt] *= alpha;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        bf16x8_t pf[2][2];
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int qh = 0; qh < 2; ++qh) {
                f32x4_t a, c;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] = fast_exp2(fmaf(st[mt][8 * qh + i], scale_log2, -m_use));
                    c[i] = fast_exp2(fmaf(st[mt][8 * qh + 4 + i], scale_log2, -m_use));
                    psum += a[i] + c[i];
                }
                pf[mt][qh] = pack_bf16x8(a, c);
            }
        l_run += psum;

        // O^T += V^T P^T: k-step (mt, qh) covers keys 32*mt + 16*qh + {4h..4h+3, 8+4h..8+4h+3}.
        const int i16 = lane & 15, nh = n >> 4;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int qh = 0; qh < 2; ++qh) {
                    const __bf16 *p0 = &Vs[cur][(32 * mt + 16 * qh + 4 * h + (i16 >> 2)) * C::VSTRIDE + dt * 32 +
                                               16 * nh + 4 * (i16 & 3)];
                    const bf16x4_t lo = lds_read_tr16(p0);
                    const bf16x4_t hi = lds_read_tr16(p0 + 8 * C::VSTRIDE);
                    acc[dt] = mfma32x32x16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pf[mt][qh],
                                           acc[dt]);
                }

        if (more)
            lstore(cur ^ 1, j + 1, kr, vr);
    }

    // Epilogue: lane holds O^T[dt*32 + 8*m0 + 4*h + m1][row]; 4 consecutive d per (dt, m0).
    l_run += __shfl_xor(l_run, 32, 64);
    if (!row_ok)
        return;
    const float inv = 1.f / l_run;
    __bf16 *dst = out + qrow * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int m0 = 0; m0 < 4; ++m0) {
            u32x2_t u = {pack_bf16x2(acc[dt][4 * m0] * inv, acc[dt][4 * m0 + 1] * inv),
                         pack_bf16x2(acc[dt][4 * m0 + 2] * inv, acc[dt][4 * m0 + 3] * inv)};
            *reinterpret_cast<u32x2_t *>(dst + dt * 32 + 8 * m0) = u;
        }
}

template <int D>
hipError_t launch_mfma(const PrefillArgs &a)
{
    const int r = a.H / a.G;
    const int QT = kPfRows / r;
    const int nqt = (a.T + QT - 1) / QT;
    const float scale_log2 = kLog2e / sqrtf((float)D);
    prefill_bf16_kernel<D><<<dim3(nqt, a.G, a.B), 256, 0, a.stream>>>(
        static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), static_cast<const __bf16 *>(a.v), a.T,
        a.H, a.G, r, QT, a.causal, scale_log2, static_cast<__bf16 *>(a.out));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, gqa_dtype dtype)
{
    if (dtype == GQA_FP32)
        return launch_rows<float>(a);
    if (a.H / a.G > kPfRows)
        return launch_rows<__bf16>(a);
    return a.D == 64 ? launch_mfma<64>(a) : launch_mfma<128>(a);
}

}  // namespace gqa
