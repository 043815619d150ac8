// prefill.hip -- GQA prefill (every position of a sequence is a query).
//
// out[b,t,h,:] = sum_{s in keys(t)} softmax_s(q[b,t,h,:] . k[b,s,g,:] / sqrt(d_h)) v[b,s,g,:]
// with g = h / r and keys(t) = [0, t] when causal, [0, T) otherwise
// ("Grouped-Query Attention" (llm-arch-kb), section 3 Reference
// implementation: broadcast of each key/value head to its H/G query heads,
// scores over sqrt(d_h), causal mask, softmax over keys, times v).
//
// 16-bit MFMA kernel, bf16 or fp16 storage (flash-attention style, one pass
// over keys with an online softmax; the score matrix never leaves registers):
//  * Workgroup = (query tile, key/value group g, sequence b). Its 256 query
//    rows are (token, head) pairs: QT = 256 / r consecutive tokens times the r
//    heads of group g, so one K/V tile in LDS serves all heads of the group
//    (the broadcast of the sketch costs no extra memory traffic).
//  * 8 waves x 32 rows. Scores are computed transposed, S^T = K . Q^T, with
//    32x32x16 bf16 MFMAs (keys in M, query rows in N): the result layout (a
//    lane holds 16 keys of one row) is directly the B operand P^T of
//    O^T = V^T . P^T, so P stays in registers.
//  * K/V tiles of 64 positions are double-buffered in LDS and loaded straight
//    from global memory into LDS (buffer_load_dwordx4 ... lds, no staging
//    registers; the buffer bounds turn rows past the sequence end into
//    zeros). Rows are unpadded with XOR-swizzled 16-byte chunks so that the
//    16-byte K reads and the V^T transposing reads (ds_read_b64_tr_b16) avoid
//    bank conflicts.
//  * Software pipeline over key tiles: while the matrix cores compute the
//    scores of tile j+1, the vector ALUs turn the scores of tile j into
//    probabilities; while they compute P_j V_j, the ALUs take the row maxima
//    of tile j+1. Each pair of probabilities goes through its FMA, its
//    exponential and its pack in three consecutive steps, so no vector
//    instruction waits on the one just before it. K runs one tile ahead of
//    V, so each load has a whole iteration to land.
//  * Causal: a query tile only visits key tiles up to its last token; the
//    heaviest tiles are launched first. Workgroups are numbered so that each
//    XCD (workgroup i runs on XCD i % 8) takes a contiguous run of query
//    tiles of the same (sequence, group): they read the same K/V prefix
//    through one L2.
//  * Softmax in base 2 against a lazily moved per-row reference (rescaling
//    only when a row maximum grows by more than 2^8): p = 2^(s*c - m) from
//    the fp32 score s with c = log2(e)/sqrt(d_h), one FMA per score (q is
//    never scaled in 16 bits); masking only on the tiles that cross the
//    causal diagonal, a window edge or the sequence end.
//
// Row kernel (fp32 path, and groups of more than 256 query heads): one
// wavefront per (b, t, h) row, lanes split d_h, online softmax over the keys
// one position at a time, fp32 arithmetic.
#include <type_traits>

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
    return bits_to_f32<__bf16>(*reinterpret_cast<const uint16_t *>(p));
}
template <>
__device__ __forceinline__ float ld<_Float16>(const _Float16 *p)
{
    return (float)*p;
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
    *reinterpret_cast<uint16_t *>(p) = (uint16_t)(pack2<__bf16>(x, 0.f) & 0xffffu);
}
template <>
__device__ __forceinline__ void st<_Float16>(_Float16 *p, float x)
{
    *reinterpret_cast<uint16_t *>(p) = (uint16_t)(pack2<_Float16>(x, 0.f) & 0xffffu);
}

template <typename T, int D>
__global__ void __launch_bounds__(64)
prefill_row_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, int T_, int H,
                   int G, int causal, int window, double scale, T *__restrict__ out)
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
    const int s0 = (causal && window > 0) ? max(0, t + 1 - window) : 0;  // first admissible key
    float qv[J], acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        qv[j] = ld(q + row * D + lane + 64 * j);
        acc[j] = 0.f;
    }
    // Scores and the running maximum in fp64: the exponent argument s - m
    // then keeps fp32 accuracy however large the scores are (an fp32 score
    // of magnitude 100 is only good to about 4e-6 in the exponent).
    double m = -INFINITY;
    float l = 0.f;
    for (int s = s0; s < nkeys; ++s) {
        if (!GQA_IN_RANGE(s, T_, 3))
            continue;
        const int64_t off = ((b * T_ + s) * G + g) * D;
        double dot = 0.0;
#pragma unroll
        for (int j = 0; j < J; ++j)
            dot += (double)qv[j] * (double)ld(k + off + lane + 64 * j);
        const double sc = wave_sum(dot) * scale;
        const double m_new = fmax(m, sc);
        const float alpha = expf((float)(m - m_new));
        const float p = expf((float)(sc - m_new));
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
    const double scale = 1.0 / sqrt((double)a.D);
    if (a.D == 64)
        prefill_row_kernel<T, 64><<<dim3((unsigned)rows), 64, 0, a.stream>>>(
            static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v), a.T, a.H, a.G,
            a.causal, a.window, scale, static_cast<T *>(a.out));
    else
        prefill_row_kernel<T, 128><<<dim3((unsigned)rows), 64, 0, a.stream>>>(
            static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v), a.T, a.H, a.G,
            a.causal, a.window, scale, static_cast<T *>(a.out));
    return hipGetLastError();
}

constexpr int kPfBN = 64;    // key/value positions per tile
constexpr int kPfWaves = 8;             // waves per workgroup, 32 query rows each
constexpr int kPfRows = 32 * kPfWaves;  // query rows per workgroup
static_assert(kPfRows == kPrefillRows, "the host's launch checks assume this row count");

template <int D>
struct PfCfg {
    static constexpr int KS = D / 16;                     // QK k-steps over d_h
    static constexpr int DT = D / 32;                     // 32-wide d tiles of O^T
    static constexpr int CH = D / 8;                      // 16-byte chunks per row
    static constexpr int WAVE_ROWS = 64 / CH;             // rows one wave load instruction fills
    static constexpr int LOADS = kPfBN / (kPfWaves * WAVE_ROWS); // load instructions per tensor per wave
    static constexpr int TILE_ELEMS = kPfBN * D;          // unpadded rows, chunks swizzled
};

// LDS tile layout: rows of d_h elements without padding; the 16-byte chunk c
// of row r sits at chunk slot c ^ kswz(r) (K) or c ^ vswz(r) (V). K is read
// 16 rows at a time at one chunk (b128 reads): r mod 16 spreads them over 16
// slots. V is read by the transposing loads, whose 32-lane halves take 4
// rows x 4 chunks (64 bytes per row) at once: with 256-byte rows (d_h = 128)
// vswz = 4*(r mod 4) puts the 4 rows in 4 different 64-byte bank ranges (with
// 2*(r mod 4), measured, half of all V-read cycles were bank conflicts); with
// 128-byte rows (d_h = 64) consecutive rows already alternate bank halves and
// vswz = 2*(r mod 4) separates the rest.
template <int D>
struct PfSwz {
    static __device__ __forceinline__ int k(int r) { return r & (D / 8 - 1); }
    static __device__ __forceinline__ int v(int r) { return D >= 128 ? (r & 3) << 2 : (r & 3) << 1; }
};

__device__ __forceinline__ u32x4_t ld16(const __bf16 *p)
{
    return *reinterpret_cast<const u32x4_t *>(p);
}


// Software pipeline over key tiles, one barrier per tile. Iteration j holds
// the scores S_j of tile j in registers and, in one basic block, computes
//   P_j = exp2(S_j * c - m)      (VALU)   while   S_{j+1} = K_{j+1} Q^T  (MFMA)
//   O  += V_j^T P_j^T            (MFMA)   while   row max of S_{j+1}     (VALU)
// so the matrix cores and the vector ALUs work on different tiles at once.
// K is read one tile ahead of V, so the buffers are staggered: iteration j
// reads K_{j+1} and V_j and loads K_{j+2} and V_{j+1} into the buffers that
// held K_j and V_{j-1}.
// E: 16-bit storage type (__bf16 or _Float16); the pointers carry its raw bits.
template <typename E, int D, bool WIN>
__global__ void __launch_bounds__(64 * kPfWaves, 8 / kPfWaves)
prefill_mfma_kernel(const __bf16 *__restrict__ q, const __bf16 *kp, const __bf16 *vp, int T, int H, int G, int r,
                    int QT, int causal, int window, float scale_log2, __bf16 *__restrict__ out)
{
    using C = PfCfg<D>;
    using SW = PfSwz<D>;
    // Four separate LDS arrays (not one [2][...] array): the compiler then
    // knows that reading one buffer does not touch another, so reads of the
    // current tiles need not wait for the direct-to-LDS loads of the next.
    __shared__ __attribute__((aligned(256))) __bf16 Ks0[C::TILE_ELEMS];
    __shared__ __attribute__((aligned(256))) __bf16 Ks1[C::TILE_ELEMS];
    __shared__ __attribute__((aligned(256))) __bf16 Vs0[C::TILE_ELEMS];
    __shared__ __attribute__((aligned(256))) __bf16 Vs1[C::TILE_ELEMS];
    auto kbuf = [&](auto i) -> __bf16 * {
        if constexpr (decltype(i)::value == 0)
            return Ks0;
        else
            return Ks1;
    };
    auto vbuf = [&](auto i) -> __bf16 * {
        if constexpr (decltype(i)::value == 0)
            return Vs0;
        else
            return Vs1;
    };

    // Workgroup i of a launch runs on XCD i % 8. Give every XCD a contiguous
    // range of work items, so that the query tiles of one (sequence, group),
    // which read the same K/V prefix, share an L2.
    const int nx = gridDim.x, ny = gridDim.y;
    const int total = nx * ny * gridDim.z;
    const int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const int item = (total % 8 == 0) ? (lin % 8) * (total / 8) + lin / 8 : lin;
    const int qt = nx - 1 - item % nx;  // heaviest causal tiles first
    const int g = (item / nx) % ny, b = item / (nx * ny);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int t0 = qt * QT;

    // This lane's query row: column n of the wave's S^T column tile.
    const int rho = wave * 32 + n;
    const int tq = t0 + rho / r;
    const bool row_ok = rho < QT * r && tq < T;
    const int64_t qrow = ((int64_t)b * T + min(tq, T - 1)) * H + g * r + rho % r;
    const int t_row_min = t0 + (wave * 32) / r;  // first query token of this wave
    const int t_row_max = min(T - 1, t0 + min(wave * 32 + 31, QT * r - 1) / r);  // last one

    // Q^T as the B operand, exactly as stored: lane holds q[row][16*ks + 8*h
    // .. +7]. The scale is applied to the fp32 scores (folded into the
    // exponent's argument), never to q: rounding q*c to 16 bits would put a
    // relative error of 2^-9 on every score, which large scores (queries
    // scaled by 16, as outlier features can be) turn into errors of 0.1 in
    // the output.
    bf16x8_t qf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        u32x4_t x = {0, 0, 0, 0};
        if (row_ok && GQA_IN_RANGE(qrow, (int64_t)gridDim.z * T * H, 0))
            x = ld16(q + qrow * D + ks * 16 + h * 8);
        qf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }

    const int t_hi = min(T, t0 + QT);
    const int kv_end = causal ? t_hi : T;
    const int ntiles = (kv_end + kPfBN - 1) / kPfBN;
    // Tiles below j_mask need no mask for any row of the workgroup.
    const int j_mask = causal ? t0 / kPfBN : T / kPfBN;
    // With a sliding window (causal only), row t sees keys [t + 1 - window, t]:
    // the workgroup starts at the first key tile any of its rows needs, and
    // tiles below j_left may hold keys left of some row's window.
    if constexpr (!WIN)
        window = 0;
    const int j_lo = WIN ? max(0, t0 + 1 - window) / kPfBN : 0;
    const int j_left = WIN ? max(j_lo, (max(0, t_hi - window) + kPfBN - 1) / kPfBN) : 0;
    const int nrel = ntiles - j_lo;  // tiles visited: relative tile i is key tile j_lo + i

    // Tile loads go straight from global memory into LDS
    // (buffer_load_dwordx4 ... lds): lane i of a wave instruction fills the
    // 16-byte LDS slot base + 16*i, i.e. row WAVE_ROWS*instr + i/CH, slot
    // i%CH, so it fetches the global chunk that the swizzle puts in that slot.
    // The buffer resource spans the tile's positions inside the sequence, so
    // rows past the sequence end read as zeros (their scores are masked to
    // -inf and their p is 0). The swizzle of a lane's rows does not depend on
    // the instruction, so one per-lane offset serves all of them.
    static_assert((kPfWaves * C::WAVE_ROWS) % C::CH == 0, "swizzle must repeat every instruction");
    const int tok_bytes = G * D * 2;
    const int rl0 = wave * C::WAVE_ROWS + lane / C::CH;  // tile row of this lane's first load
    const int sslot = lane % C::CH;
    const int voff_k = rl0 * tok_bytes + g * D * 2 + (sslot ^ SW::k(rl0)) * 16;
    const int voff_v = rl0 * tok_bytes + g * D * 2 + (sslot ^ SW::v(rl0)) * 16;
    auto load_tile = [&](const __bf16 *src, __bf16 *dst, int tile, bool is_v) {
        const int row0 = tile * kPfBN;
        const __bf16 *base = src + ((int64_t)b * T + row0) * G * D;
        const int nrec = (min(T, row0 + kPfBN) - row0) * tok_bytes;
        if (GQA_IN_RANGE(row0, T, 1) && GQA_IN_RANGE(b, gridDim.z, 1))
            buffer_rows_to_lds<C::LOADS>(base, nrec, dst + wave * C::WAVE_ROWS * D, kPfWaves * C::WAVE_ROWS * D,
                                         is_v ? voff_v : voff_k, kPfWaves * C::WAVE_ROWS * tok_bytes);
    };

    // LDS fragment addresses. The swizzles only permute chunks inside a
    // row, and the chunk index splits into bits that vary per read and bits
    // fixed per lane, so an address is a per-lane base XOR a constant
    // (buffers are 256-byte aligned, rows 2*d_h bytes):
    //  * K fragment (A operand of S^T = K Q^T) for k-step ks of M tile mt:
    //    lane (n, h) reads chunk 2*ks + h of key row 32*mt + n, stored at slot
    //    (2*ks) ^ (h ^ kswz(n)) (kswz(n + 32) = kswz(n)).
    //  * V^T fragment (A operand of O^T = V^T P^T) for key k-step kstep and d
    //    tile dt: keys 16*kstep + {4h..4h+3, 8+4h..8+4h+3}; lane reads row
    //    16*kstep + 4*h + i16/4 (and 8 rows on), columns dt*32 + 16*nh +
    //    4*(i16%4) .. +3, i.e. chunk 4*dt + x with x = 2*nh + (i16%4)/2, half
    //    (i16%2), stored at slot (4*dt) ^ (x ^ vswz(row)) (vswz depends on
    //    row % 4 only).
    static_assert(D * 2 >= 128, "row must hold the XOR-ed bits");
    const int i16 = lane & 15, nh = n >> 4;
    const uint32_t kb_lane = n * D * 2 + ((h ^ SW::k(n)) * 16);
    const int vrow = 4 * h + (i16 >> 2);
    const uint32_t vb_lane =
        vrow * D * 2 + (((2 * nh + ((i16 & 3) >> 1)) ^ SW::v(vrow)) * 16) + (i16 & 1) * 8;
    auto kfrag = [&](const __bf16 *Kc, int ks, int mt) {
        const char *a = (const char *)Kc + (kb_lane ^ (uint32_t)(32 * ks)) + mt * 32 * D * 2;
        return __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)a);
    };
    auto vfrag = [&](const __bf16 *Vc, int kstep, int dt) {
        const char *a = (const char *)Vc + (vb_lane ^ (uint32_t)(64 * dt)) + kstep * 16 * D * 2;
        const bf16x4_t lo = lds_read_tr16((const __bf16 *)a);
        const bf16x4_t hi = lds_read_tr16((const __bf16 *)(a + 8 * D * 2));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    // S^T = K Q^T for one tile (plain order): two 32-key M tiles.
    auto qk = [&](const __bf16 *Kc, f32x16_t (&st)[2]) {
        st[0] = st[1] = (f32x16_t){};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            st[0] = mfma32x32x16<E>(kfrag(Kc, ks, 0), qf[ks], st[0]);
            st[1] = mfma32x32x16<E>(kfrag(Kc, ks, 1), qf[ks], st[1]);
        }
    };

    // Register v of S^T tile mt holds key tile*64 + 32*mt + 8*(v/4) + 4*h + v%4.
    auto mask = [&](f32x16_t (&st)[2], int tile) {
        const int tile_last = tile * kPfBN + kPfBN - 1;
        const bool need_right = causal ? (tile_last > t_row_min) : (tile_last >= T);
        const bool need_left = WIN && tile * kPfBN < t_row_max + 1 - window;
        if (!need_right && !need_left)
            return;
        const int key_lim = causal ? tq : T - 1;             // last admissible key
        const int key_lo = WIN ? tq + 1 - window : 0;  // first admissible key
        const int tk0 = tile * kPfBN + 4 * h;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tk = tk0 + 32 * mt + 8 * (v >> 2) + (v & 3);
                st[mt][v] = (tk <= key_lim && tk >= key_lo) ? st[mt][v] : -INFINITY;
            }
    };

    // Online softmax in base 2 with a lazily moved reference m_run (in
    // scaled units): registers hold the raw scores s (fp32) and p =
    // 2^(s*c - m_run) with c = scale*log2(e), one FMA and one exponential per
    // score. The reference only moves when a row maximum exceeds it by more
    // than kLazy, so p <= 2^kLazy; softmax is unchanged by the choice of
    // reference. A move by delta found on tile j+1 applies to the
    // probabilities of tile j+1 on, and rescales O and l by 2^-delta at the
    // start of the next iteration, after P_j V_j has been added.
    constexpr float kLazy = 8.f;
    float m_run = 0.f, l_run = 0.f, alpha = 1.f;
    bool move = false;
    bool m_set = false;  // a finite reference exists (a window may hide every key of the first tile)
    // maximum() (NaN-propagating) maps to three-input v_maximum3 without the
    // operand canonicalisation that fmaxf costs.
    auto max_part = [&](const f32x16_t (&st)[2], int v, float &mx0, float &mx1) {
        mx0 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx0, st[0][v]), st[0][v + 1]);
        mx1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx1, st[1][v]), st[1][v + 1]);
    };
    float delta = 0.f;
    auto max_finish = [&](float mx0, float mx1) {
        float mx = __builtin_elementwise_maximum(mx0, mx1);
        {
            float a, b;
            xor_pair<32>(mx, a, b);  // VALU lane swap: does not queue behind LDS reads
            mx = __builtin_elementwise_maximum(a, b);
        }
        mx = fmaf(mx, scale_log2, -m_run);  // scaled, relative to m_run (-inf stays -inf)
        const bool first = WIN && !m_set && mx != -INFINITY;  // O and l are still zero
        move = mx > kLazy || first;
        delta = move ? mx : 0.f;
        alpha = first ? 0.f : fast_exp2(-delta);
        m_set = m_set || first;
        m_run += delta;
    };
    auto row_max = [&](const f32x16_t (&st)[2]) {
        float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; v += 2)
            max_part(st, v, mx0, mx1);
        max_finish(mx0, mx1);
    };

    // The row sum adds the bf16-rounded p that the P V product uses (dot
    // product with (1, 1)). One word in one go, for the plain iterations.
    // Word w (0..15) of P_j: the bf16 pair for scores st[mt][8*qh + 2*i],
    // +1 (kk = w/4 = 2*mt + qh, i = w%4), word i of pw[kk].
    auto p_word = [&](const f32x16_t (&st)[2], int w, u32x4_t (&pw)[4], float &ps0, float &ps1) {
        const int kk = w >> 2, i = w & 3, mt = kk >> 1, qh = kk & 1;
        const float e0 = fast_exp2(fmaf(st[mt][8 * qh + 2 * i], scale_log2, -m_run));
        const float e1 = fast_exp2(fmaf(st[mt][8 * qh + 2 * i + 1], scale_log2, -m_run));
        const uint32_t x = pack2<E>(e0, e1);
        pw[kk][i] = x;
        float &ps = (w & 1) ? ps1 : ps0;
        ps = add_pair<E>(x, ps);
    };

    // Step in which word w of P_j starts (its FMAs); its pack lands two steps
    // later, before the P V step that reads its word group.
    constexpr auto p_slot = [](int w) {
        if constexpr (D == 128)
            return w < 4 ? w / 2 : w - 2;
        else
            return w / 2;
    };
    static_assert([p_slot] {
        for (int w = 0; w < 16; ++w)
            if (!(p_slot(w) + 2 < C::KS + C::DT * (w / 4)))
                return false;
        return true;
    }(), "every word is packed before the P V step that reads it");
    // The same words in three stages spread over consecutive steps of the
    // pipelined iteration: the two FMAs of word w in step p_slot(w), its two
    // exponentials in the next step and its pack and row-sum add in the one
    // after (steps 0..KS-1 are the QK steps, KS + s the P V steps). No
    // instruction then waits on a result issued just before it, which in
    // this in-order wave would also hold back the next MFMA. Scores are
    // turned into probabilities in place.
    auto p_stage = [&](f32x16_t (&s)[2], int slot, u32x4_t (&pw)[4]) {
#pragma unroll
        for (int w = 0; w < 16; ++w)
            if (p_slot(w) + 2 == slot)
                pw[w >> 2][w & 3] = pack2<E>(s[w >> 3][8 * ((w >> 2) & 1) + 2 * (w & 3)],
                                             s[w >> 3][8 * ((w >> 2) & 1) + 2 * (w & 3) + 1]);
#pragma unroll
        for (int w = 0; w < 16; ++w)
            if (p_slot(w) + 1 == slot) {
                const int v0 = 8 * ((w >> 2) & 1) + 2 * (w & 3);
                s[w >> 3][v0] = fast_exp2(s[w >> 3][v0]);
                s[w >> 3][v0 + 1] = fast_exp2(s[w >> 3][v0 + 1]);
            }
#pragma unroll
        for (int w = 0; w < 16; ++w)
            if (p_slot(w) == slot) {
                const int v0 = 8 * ((w >> 2) & 1) + 2 * (w & 3);
                s[w >> 3][v0] = fmaf(s[w >> 3][v0], scale_log2, -m_run);
                s[w >> 3][v0 + 1] = fmaf(s[w >> 3][v0 + 1], scale_log2, -m_run);
            }
    };

    f32x16_t acc[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
        acc[dt] = (f32x16_t){};

    auto rescale = [&]() {
        if (__any(move)) {
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
                acc[dt] *= alpha;
        }
    };

    f32x16_t st[2][2];  // S_j lives in st[j % 2]

    // Iteration j < ntiles - 1; P = j % 2 selects the buffers. The body is
    // laid out by hand in steps fenced with sched_barrier: each QK step
    // issues the K reads of the next step, two MFMAs and a chunk of the
    // softmax of S_j; each P V step issues the V^T reads of the next step,
    // one MFMA, the last stages of P_j's words and part of the row maximum
    // of S_{j+1}, then (when a step is left) the reference update; the row
    // sums of P_j follow the last P V step.
    constexpr int kPfDist = 2;  // LDS fragment reads run this many steps ahead
    constexpr int kPvSteps = 4 * C::DT;
    // P_j words go through p_stage in every step; the row max of S_{j+1}
    // takes 8 P V steps from kMaxStart, late enough for the last QK MFMAs
    // (d_h = 128: after the P V steps that still carry most of P_j's words).
    constexpr int kMaxStart = D == 128 ? 6 : (kPvSteps >= 12 ? 4 : 0);
    static_assert(kMaxStart + 8 <= kPvSteps, "row max takes 8 steps");
    constexpr bool kEarlyFinish = kMaxStart + 8 < kPvSteps;  // a P V step is left after the maximum
    auto iter = [&](auto P, int j) {
        constexpr int p = decltype(P)::value;
        wait_vector_memory();  // this wave's loads of K_{j+1} and V_j have landed
        __syncthreads();       // everyone's have; every wave is done with K_j and V_{j-1}
        if (j + 2 < nrel)
            load_tile(kp, kbuf(Ic<p>{}), j_lo + j + 2, false);
        load_tile(vp, vbuf(Ic<1 - p>{}), j_lo + j + 1, true);
        rescale();
        const __bf16 *Kc = kbuf(Ic<1 - p>{});
        const __bf16 *Vc = vbuf(Ic<p>{});
        f32x16_t(&sc)[2] = st[p];
        f32x16_t(&sn)[2] = st[1 - p];
        u32x4_t pw[4];
        __builtin_amdgcn_sched_barrier(0);

        // Fragments are read kPfDist steps ahead of their MFMA; inside a step
        // the reads go first, then each MFMA followed by its share of VALU.
        bf16x8_t kf[C::KS][2];
#pragma unroll
        for (int i = 0; i < kPfDist && i < C::KS; ++i) {
            kf[i][0] = kfrag(Kc, i, 0);
            kf[i][1] = kfrag(Kc, i, 1);
        }
        sn[0] = sn[1] = (f32x16_t){};
        __builtin_amdgcn_sched_barrier(0);
        // The QK steps carry most of the exponentials: when both waves of a
        // SIMD compete for issue, the one in its QK steps goes first
        // (measured: 1-2% faster than equal priority).
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            if (ks + kPfDist < C::KS) {
                kf[ks + kPfDist][0] = kfrag(Kc, ks + kPfDist, 0);
                kf[ks + kPfDist][1] = kfrag(Kc, ks + kPfDist, 1);
            }
            sn[0] = mfma32x32x16<E>(kf[ks][0], qf[ks], sn[0]);
            sn[1] = mfma32x32x16<E>(kf[ks][1], qf[ks], sn[1]);
            p_stage(sc, ks, pw);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x402, 32 / C::KS, 0);  // VALU incl. transcendental
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 32 / C::KS, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        float mx0 = -INFINITY, mx1 = -INFINITY;
        bf16x8_t vf[kPvSteps];
#pragma unroll
        for (int i = 0; i < kPfDist; ++i)
            vf[i] = vfrag(Vc, i / C::DT, i % C::DT);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < kPvSteps; ++s) {
            const int kstep = s / C::DT, dt = s % C::DT;
            if (s + kPfDist < kPvSteps)
                vf[s + kPfDist] = vfrag(Vc, (s + kPfDist) / C::DT, (s + kPfDist) % C::DT);
            acc[dt] = mfma32x32x16<E>(vf[s], __builtin_bit_cast(bf16x8_t, pw[kstep]), acc[dt]);
            p_stage(sc, C::KS + s, pw);
            if (s >= kMaxStart && s < kMaxStart + 8)
                max_part(sn, 2 * (s - kMaxStart), mx0, mx1);
            if (kEarlyFinish && s == kMaxStart + 8) {
                // The reference update goes right after the last maximum
                // step, so its cross-lane exchange overlaps the remaining
                // MFMAs; the empty asm keeps the compiler from sinking it to
                // the end of the iteration (measured: about 1.5% faster).
                max_finish(mx0, mx1);
                asm volatile("" : "+v"(delta), "+v"(alpha));
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Row sums after the last P V step: inside the MFMA steps these 16
        // adds cost more issue time than here (measured 6% slower per call).
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            float &ps = (w & 1) ? ps1 : ps0;
            ps = add_pair<E>(pw[w >> 2][w & 3], ps);
        }
        l_run += ps0 + ps1;
        if constexpr (!kEarlyFinish)
            max_finish(mx0, mx1);
    };
    // Plain iterations (the tile after them needs a mask, or none follows):
    // program order, buffers picked at run time, S_j kept in st[0].
    auto tail = [&](int j) {
        const bool odd = j & 1;
        wait_vector_memory();
        __syncthreads();
        const bool more = j + 1 < nrel;
        if (more) {
            if (j + 2 < nrel)
                load_tile(kp, odd ? Ks1 : Ks0, j_lo + j + 2, false);
            load_tile(vp, odd ? Vs0 : Vs1, j_lo + j + 1, true);
        }
        rescale();
        u32x4_t pw[4];
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int w = 0; w < 16; ++w)
            p_word(st[0], w, pw, ps0, ps1);
        l_run += ps0 + ps1;
        const __bf16 *Vc = odd ? Vs1 : Vs0;
#pragma unroll
        for (int s = 0; s < kPvSteps; ++s)
            acc[s % C::DT] = mfma32x32x16<E>(vfrag(Vc, s / C::DT, s % C::DT),
                                          __builtin_bit_cast(bf16x8_t, pw[s / C::DT]), acc[s % C::DT]);
        if (more) {
            qk(odd ? Ks0 : Ks1, st[0]);
            mask(st[0], j_lo + j + 1);
            row_max(st[0]);
        }
    };

    // Prologue: K_0, V_0 and K_1 in flight, S_0 computed (relative tiles).
    load_tile(kp, Ks0, j_lo, false);
    load_tile(vp, Vs0, j_lo, true);
    if (nrel > 1)
        load_tile(kp, Ks1, j_lo + 1, false);
    wait_vector_memory();
    __syncthreads();
    qk(Ks0, st[0]);
    mask(st[0], j_lo);
    {
        // The first reference is the row maximum of the first tile. Without a
        // window that tile holds key 0, admissible for every row; with one, a
        // row may see no key of it, and its reference is set on its first
        // admissible tile instead.
        float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; v += 2)
            max_part(st[0], v, mx0, mx1);
        float mx = __builtin_elementwise_maximum(mx0, mx1);
        {
            float a, b;
            xor_pair<32>(mx, a, b);  // VALU lane swap: does not queue behind LDS reads
            mx = __builtin_elementwise_maximum(a, b);
        }
        m_set = mx != -INFINITY;
        m_run = m_set ? mx * scale_log2 : 0.f;
    }

    // Relative iteration j computes key tile j_lo + j + 1; the pipelined body
    // runs while that tile needs no mask (j_left <= j_lo + j + 1 < j_mask),
    // starting at an even j so that the buffer parity is known statically.
    int f0 = max(0, j_left - j_lo - 1);
    f0 += f0 & 1;
    int f1 = min(nrel - 1, j_mask - j_lo - 1);
    if (f1 <= f0)
        f0 = f1 = 0;
    int j = 0;
    for (; j < f0; ++j)
        tail(j);
    for (; j + 1 < f1; j += 2) {
        iter(Ic<0>{}, j);
        iter(Ic<1>{}, j + 1);
    }
    if (j < f1) {
        iter(Ic<0>{}, j);
        ++j;
        st[0][0] = st[1][0];
        st[0][1] = st[1][1];
    }
    for (; j < nrel; ++j)
        tail(j);

    // Epilogue: lane holds O^T[dt*32 + 8*m0 + 4*h + m1][row]; 4 consecutive d per (dt, m0).
    const float lsum = xor_add<32>(l_run);
    if (!row_ok || !GQA_IN_RANGE(qrow, (int64_t)gridDim.z * T * H, 2))
        return;
    const float inv = 1.f / lsum;
    __bf16 *dst = out + qrow * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int m0 = 0; m0 < 4; ++m0) {
            u32x2_t u = {pack2<E>(acc[dt][4 * m0] * inv, acc[dt][4 * m0 + 1] * inv),
                         pack2<E>(acc[dt][4 * m0 + 2] * inv, acc[dt][4 * m0 + 3] * inv)};
            *reinterpret_cast<u32x2_t *>(dst + dt * 32 + 8 * m0) = u;
        }
}

template <typename E, int D, bool WIN>
hipError_t launch_mfma(const PrefillArgs &a)
{
    const int r = a.H / a.G;
    const int QT = kPfRows / r;
    const int nqt = (a.T + QT - 1) / QT;
    const float scale_log2 = kLog2e / sqrtf((float)D);
    prefill_mfma_kernel<E, D, WIN><<<dim3(nqt, a.G, a.B), 64 * kPfWaves, 0, a.stream>>>(
        static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k), static_cast<const __bf16 *>(a.v), a.T,
        a.H, a.G, r, QT, a.causal, a.window, scale_log2, static_cast<__bf16 *>(a.out));
    return hipGetLastError();
}

template <typename E>
hipError_t launch_16bit(const PrefillArgs &a)
{
    if (a.H / a.G > kPfRows)
        return launch_rows<E>(a);
    if (a.window > 0)
        return a.D == 64 ? launch_mfma<E, 64, true>(a) : launch_mfma<E, 128, true>(a);
    return a.D == 64 ? launch_mfma<E, 64, false>(a) : launch_mfma<E, 128, false>(a);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, gqa_dtype dtype)
{
    if (dtype == GQA_FP32)
        return launch_rows<float>(a);
    if (dtype == GQA_FP16)
        return launch_16bit<_Float16>(a);
    return launch_16bit<__bf16>(a);
}

GQA_DEBUG_READER(debug_take_prefill)

}  // namespace gqa
