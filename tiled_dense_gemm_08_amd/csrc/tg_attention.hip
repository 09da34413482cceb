// tg_attention.hip — fused scaled dot-product attention (forward) for gfx950.
//
// The block-wise form the lqnn.cn TileLang walkthrough (section 3.2) and the
// xdnf.cn article (section 3.2) describe: K and V are loaded tile by tile
// into LDS by the same global->LDS copies and two-stage ring as the GEMM,
// each tile's scores are multiplied on the matrix cores, and the softmax is
// folded in online, in registers, before the next tile:
//     m' = max(m, max_j s_j)          alpha = exp(m - m')
//     l' = alpha l + sum_j exp(s_j - m')
//     O' = alpha O + sum_j exp(s_j - m') V_j
// and at the end O / l and lse = m + log l.  Scores and the softmax are fp32,
// the weights are rounded to fp16 for the second product, O is stored fp16.
//
// Work split: a workgroup of 8 waves owns 256 queries of one (batch, head);
// each wave owns 32 of them and loops over the keys in tiles of 64.  Every
// K and V tile is copied to LDS once for the 256 queries (with 4 waves and
// 128 queries the kernel ran 3-4 % slower: twice the copies per query).
//
// Both products are computed transposed so that a lane owns one query:
//  * scores S^T = K . Q^T on v_mfma_f32_32x32x16_f16 with K from LDS (first
//    source, rows = keys) and the wave's Q fragments in registers (second
//    source, columns = queries): lane l holds query l % 32 and, in register
//    r of a 32-key tile, key 8 (r / 4) + 4 (l / 32) + r % 4.  A row's maximum
//    is the maximum over the lane's registers and lane l ^ 32.
//  * O^T = V^T . P^T with V^T read from the LDS tile by transpose reads
//    (first source, rows = head dimension) and P^T straight from the score
//    registers converted to fp16 (second source): a lane's 8 weights of a
//    16-key chunk are keys {4h .. 4h+3, 8+4h .. 11+4h} (h = l / 32), and the
//    transpose reads fetch V's rows in that same order, so no weight moves
//    between lanes.  The O^T accumulator again gives lane l query l % 32, so
//    the rescale by alpha is one multiply per register.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tg_attention.h"

namespace tg {
namespace attn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));

#define TGA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr int WAVES = 8, BQ = 32 * WAVES, BKV = 64, THREADS = 64 * WAVES;

template <int D>
struct Tile {
    static constexpr int ROWB = 2 * D;           // bytes of a K or V row
    static constexpr int CHUNKS = ROWB / 16;     // 16-byte chunks per row
    static constexpr int BYTES = BKV * ROWB;     // one K or V tile
    // d = 128: the scores of tile j + 1 are computed while tile j's softmax
    // runs (K in a three-stage ring); d = 64 keeps the plain order, where the
    // fewer registers let more waves share a SIMD instead (measured faster).
    static constexpr bool PIPE = D == 128;
    static constexpr int KST = PIPE ? 3 : 2;     // K ring depth; V: two stages
    static constexpr int U = PIPE ? 2 : 1;       // tiles per unrolled loop body
    static constexpr int LDS = (KST + 2) * BYTES;
    static constexpr int LOADS = BYTES / 1024 / WAVES;   // copies per wave per tile
    static constexpr int ROWS_PER_LOAD = 1024 / ROWB;
    static constexpr int DK = D / 16;            // k-steps of the score product
    static constexpr int DT = D / 32;            // 32-row blocks of O^T
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(BYTES % (1024 * WAVES) == 0, "copy split");
};

// K tile: 32 lanes read 32 consecutive rows at one chunk (ds_read_b128);
// XOR by row % 8 spreads them over the banks.
__device__ __forceinline__ int swz_k(int row) { return row & 7; }

// V tile: a transpose read touches rows {4h + e} (e < 4, h < 2) at one
// 32-byte column pair per 16-lane group; even XOR masks keep the pairs whole
// and put the 8 rows on distinct 32-byte slots (rows of 128 bytes: 4 slots).
template <int CHUNKS>
__device__ __forceinline__ int swz_v(int row)
{
    if constexpr (CHUNKS >= 16)
        return 2 * (row & 3) + 8 * ((row >> 2) & 1);
    else
        return 2 * (row & 3);
}

__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void wait_vmcnt0()
{
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
}

// 16 bytes per lane from buffer offset voff to LDS address m0 + 16 lane (see
// the GEMM's copy: M0 is written only here, one wait state before the load).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)p;
}

// Copies of one K or V tile (keys kv0 .. kv0+63 of a head whose rows are
// rstride elements apart): wave w's instruction t fills LDS bytes
// [1 KiB (w LOADS + t), +1 KiB) = ROWS_PER_LOAD rows; lane i takes row
// i / CHUNKS and physical chunk i % CHUNKS, and fetches the logical chunk that
// the tile's swizzle puts there.  Rows at or past Lk fall outside the
// descriptor's range and read as zeros.
template <int D, bool IS_V>
__device__ __forceinline__ void copy_tile(const _Float16 *head, int64_t rstride, int kv0, int Lk,
                                          uint32_t head_bytes, uint32_t lds_tile)
{
    using T = Tile<D>;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t start = (int64_t)kv0 * rstride * 2;
    const uint32_t range = kv0 < Lk ? head_bytes - (uint32_t)start : 0;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)head + start), 0, (int)range, kRsrcWord3);
#pragma unroll
    for (int t = 0; t < T::LOADS; t++) {
        const int inst = wave * T::LOADS + t;
        const int row = inst * T::ROWS_PER_LOAD + lane / T::CHUNKS;
        const int pc = lane % T::CHUNKS;
        const int lc = pc ^ (IS_V ? swz_v<T::CHUNKS>(row) : swz_k(row));
        const uint32_t voff = (uint32_t)((int64_t)row * rstride * 2) + (uint32_t)(lc * 16);
        dma16(rsrc, voff, __builtin_amdgcn_readfirstlane(lds_tile + inst * 1024));
    }
}

struct AttnParams {
    const _Float16 *Q, *K, *V;
    _Float16 *O;
    float *lse;                 // [B][H][Lq] or nullptr
    int B, H, group, Lq, Lk;    // group = H / Hkv
    int64_t qs[3], ks[3], vs[3], os[3];   // {batch, head, row} strides, elements
    uint32_t k_bytes, v_bytes;  // descriptor range of one head's K / V rows
    float scale_log2;           // |scale| * log2(e)
    int negate_q;               // scale < 0: Q is negated on load
    int zero_q;                 // scale == 0: Q is read as zeros (uniform weights)
    int nqb;                    // query blocks per head
    int causal;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(THREADS, 1) attn_fwd(AttnParams p)
{
    using T = Tile<D>;
    __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5;        // lane half
    const int col = lane & 31;      // the lane's query within the wave

    // workgroup -> (batch, head, query block); each XCD gets a contiguous
    // range, so the query blocks of a head share that XCD's L2
    const int total = p.B * p.H * p.nqb;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int per = total >> 3, rem = total & 7;
    const int start = xcd * per + (xcd < rem ? xcd : rem);
    const int t_log = start + slot;
    int bh = t_log / p.nqb;
    int qb = t_log - bh * p.nqb;
    if constexpr (CAUSAL) {
        // longest rows first: when the XCD's range holds whole heads, walk it
        // by query block (longest first) across those heads, so that every
        // CU of the XCD starts on long work; else longest first per head
        const int cnt = per + (xcd < rem ? 1 : 0);
        if (start % p.nqb == 0 && cnt % p.nqb == 0) {
            const int heads = cnt / p.nqb;
            bh = start / p.nqb + slot % heads;
            qb = p.nqb - 1 - slot / heads;
        } else {
            qb = p.nqb - 1 - qb;
        }
    }
    const int b = bh / p.H, hq = bh - b * p.H, hk = hq / p.group;
    const int q_wg = qb * BQ;
    const int q0 = q_wg + wave * 32;      // the wave's first query
    const int query = q0 + col;
    const int shift = p.Lk - p.Lq;        // causal: key j visible to query i iff j <= i + shift

    // key tiles this workgroup needs
    int nblk = (p.Lk + BKV - 1) / BKV;
    if constexpr (CAUSAL) {
        const int last_q = min(q_wg + BQ, p.Lq) - 1;
        const int last_key = last_q + shift;
        nblk = last_key < 0 ? 0 : min(nblk, last_key / BKV + 1);
    }

    const _Float16 *Kh = p.K + b * p.ks[0] + hk * p.ks[1];
    const _Float16 *Vh = p.V + b * p.vs[0] + hk * p.vs[1];
    // K tiles in a KST-stage ring, V tiles in a two-stage ring; with the
    // pipelined order K runs two tiles ahead of V.
    const uint32_t lds0 = lds_addr(smem);
    const uint32_t lds_v = lds0 + T::KST * T::BYTES;
    if (nblk > 0) {
        copy_tile<D, false>(Kh, p.ks[2], 0, p.Lk, p.k_bytes, lds0);
        copy_tile<D, true>(Vh, p.vs[2], 0, p.Lk, p.v_bytes, lds_v);
    }
    if (T::PIPE && nblk > 1)
        copy_tile<D, false>(Kh, p.ks[2], BKV, p.Lk, p.k_bytes, lds0 + T::BYTES);

    // the wave's queries as second-source fragments: lane l holds
    // Q[query][16 ks + 8 h .. +7]
    half8 qf[T::DK];
    {
        const bool ok = query < p.Lq;
        const _Float16 *qrow = p.Q + b * p.qs[0] + hq * p.qs[1] + (int64_t)(ok ? query : 0) * p.qs[2];
        // a negative scale is applied as |scale| to -Q (negation is exact), so
        // that the scores are always scaled by a positive factor; a zero scale
        // as the factor 1 on a zero Q, so every visible score is exactly 0
#pragma unroll
        for (int ks = 0; ks < T::DK; ks++) {
            const half8 v = *(const half8 *)(qrow + 16 * ks + 8 * h);
            qf[ks] = ok && !p.zero_q ? (p.negate_q ? -v : v) : half8{};
        }
    }

    // per-lane LDS offsets of the fragment reads
    int koff[T::DK];
#pragma unroll
    for (int ks = 0; ks < T::DK; ks++)
        koff[ks] = col * T::ROWB + (((2 * ks + h) ^ swz_k(col)) * 16);
    int voff[T::DT];
    {
        const int G = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
        const int row = 4 * h + e;
        const int cg = 2 * (G & 1) + (q >> 1);
#pragma unroll
        for (int dt = 0; dt < T::DT; dt++)
            voff[dt] = row * T::ROWB + ((((4 * dt) | cg) ^ swz_v<T::CHUNKS>(row)) * 16) +
                       (q & 1) * 8;
    }

    float16v acc[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; dt++)
        acc[dt] = float16v{};
    float m = -INFINITY;   // reference maximum of the scaled scores (log2 units)
    float l = 0.f;         // the lane's share of the running sum, relative to m

    // scores of 64 keys x 32 queries (two 32-key tiles) from a K tile
    auto score_mfma = [&](const char *kt, int ks, int t, float16v &acc_s) {
        const half8 kf = *(const half8 *)(kt + koff[ks] + t * 32 * T::ROWB);
        acc_s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], acc_s, 0, 0, 0);
    };

    // Scores of the current and of the next key tile, double-buffered: the
    // pipelined loop is unrolled by two tiles, so that the two buffers trade
    // roles without register moves (and the V stage offsets are fixed).
    // Tile maximum of the raw scores of key tile jt (rows of the lane's
    // query, both halves of the wave).  Only tiles that reach past Lk or
    // across the causal diagonal of the wave's first query mask anything (a
    // uniform branch: the others skip the per-key test).
    auto tile_max = [&](float16v(&sc)[2], int jt) {
        const int kvt = jt * BKV;
        const bool edge = kvt + BKV > p.Lk || (CAUSAL && kvt + BKV - 1 > q0 + shift);
        float mxt = -INFINITY;
        if (edge) {
#pragma unroll
            for (int t = 0; t < 2; t++) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int key = kvt + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
                    const bool vis = key < p.Lk && (!CAUSAL || key <= query + shift);
                    sc[t][r] = vis ? sc[t][r] : -INFINITY;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                mxt = fmaxf(mxt, sc[t][r]);
        return fmaxf(mxt, __shfl_xor(mxt, 32));
    };

    float16v sa[2] = {float16v{}, float16v{}}, sb[2] = {float16v{}, float16v{}};
    // pipelined: the maximum of the tile whose scores are ready, taken while
    // the previous tile's second product runs
    float mx_next = -INFINITY;
    if (T::PIPE && nblk > 0) {
        wait_vmcnt0();
        lds_barrier();
#pragma unroll
        for (int ks = 0; ks < T::DK; ks++)
#pragma unroll
            for (int t = 0; t < 2; t++)
                score_mfma(smem, ks, t, sa[t]);
        mx_next = tile_max(sa, 0);
    }

    // key tile j, where J = j mod U
    auto step = [&](auto jc, int j) {
        constexpr int J = decltype(jc)::value;
        const int JV = T::U == 2 ? J : j;   // V stage parity
        float16v(&s)[2] = (T::PIPE && (J & 1)) ? sb : sa;    // tile j's scores
        float16v(&sn)[2] = (T::PIPE && (J & 1)) ? sa : sb;   // tile j+1's (pipelined)
        if (!T::PIPE || j > 0) {
            wait_vmcnt0();
            // pipelined: K tile j+1 and V tile j in LDS; plain: K and V tile j.
            // Every wave is past the tiles the copies below overwrite.
            lds_barrier();
        }
        if constexpr (T::PIPE) {
            if (j + 2 < nblk)
                copy_tile<D, false>(Kh, p.ks[2], (j + 2) * BKV, p.Lk, p.k_bytes,
                                    lds0 + ((j + 2) % T::KST) * T::BYTES);
        } else {
            if (j + 1 < nblk)
                copy_tile<D, false>(Kh, p.ks[2], (j + 1) * BKV, p.Lk, p.k_bytes,
                                    lds0 + ((j + 1) % T::KST) * T::BYTES);
        }
        if (j + 1 < nblk)
            copy_tile<D, true>(Vh, p.vs[2], (j + 1) * BKV, p.Lk, p.v_bytes,
                               lds_v + ((JV + 1) & 1) * T::BYTES);
        const char *k_next = smem + ((j + 1) % T::KST) * T::BYTES;   // stale on the last tile
        const char *vs_tile = smem + T::KST * T::BYTES + (JV & 1) * T::BYTES;
        const int kv0 = j * BKV;
        // Causal: a tile whose first key lies past the diagonal of the wave's
        // last query is masked for every query of the wave (a wave-uniform
        // test). Its weights are all 0, so the wave skips its scores, exp2
        // and V product, which would only add zeros; so do the later tiles.
        // The wave still takes part in the copies and barriers.
        const bool dead = CAUSAL && kv0 > q0 + 31 + shift;
        const bool dead_next = CAUSAL && kv0 + BKV > q0 + 31 + shift;
        if constexpr (!T::PIPE) {
            if (!dead) {
                const char *k_tile = smem + (j % T::KST) * T::BYTES;
                s[0] = float16v{};
                s[1] = float16v{};
#pragma unroll
                for (int ks = 0; ks < T::DK; ks++)
#pragma unroll
                    for (int t = 0; t < 2; t++)
                        score_mfma(k_tile, ks, t, s[t]);
            }
        }
        if (dead) {
            if constexpr (T::PIPE)
                mx_next = -INFINITY;   // the next tile's maximum: nothing visible
            return;
        }

        const float mx = T::PIPE ? mx_next : tile_max(s, j);

        // Lazy rescale: the weights are taken relative to a reference m that
        // moves only when some row's maximum exceeds it by more than 2^8, so
        // the weights stay below 256 (exact range for fp16) and O^T and l are
        // rescaled rarely -- the first tile, and when the maximum jumps.
        // m stays -inf while a row has seen no visible key.
        const float mt = mx * p.scale_log2;          // tile maximum, log2 units
        if (__builtin_amdgcn_ballot_w64(mt > m + 8.f) != 0) {
            const float m_new = fmaxf(m, mt);
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
            for (int dt = 0; dt < T::DT; dt++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    acc[dt][r] *= alpha;
            l *= alpha;
            m = m_new;
        }
        // a row with no visible key yet has only -inf scores: weight 0
        const float m_w = m == -INFINITY ? 0.f : m;

        // The next tile's scores on the matrix cores, interleaved with this
        // tile's weights exp2(s scale log2e - m), row sum and fp16 weights
        // on the vector unit.
        half8 pf[4];
        float rs = 0.f;
        if constexpr (!T::PIPE) {
#pragma unroll
            for (int t = 0; t < 2; t++) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const float w =
                        __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], p.scale_log2, -m_w));
                    rs += w;
                    pf[2 * t + r / 8][r % 8] = (_Float16)w;
                }
            }
        } else {
            sn[0] = float16v{};
            sn[1] = float16v{};
        }
        // pipelined: 2 DK MFMAs and 32 weights, 32 / (2 DK) weights per MFMA
        // (the MFMAs left out when the next tile is dead for the wave)
        constexpr int NM = 2 * T::DK, WPM = 32 / NM;
        auto weights_and_scores = [&](auto mf) {
            constexpr bool MF = decltype(mf)::value;
            half8 kf_next = MF ? *(const half8 *)(k_next + koff[0]) : half8{};
#pragma unroll
            for (int i = 0; i < NM; i++) {
                if constexpr (MF) {
                    const int ks = i / 2, t = i % 2;
                    const half8 kf = kf_next;
                    if (i + 1 < NM)
                        kf_next = *(const half8 *)(k_next + koff[(i + 1) / 2] +
                                                   ((i + 1) % 2) * 32 * T::ROWB);
                    sn[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sn[t], 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < WPM; u++) {
                    const int e = i * WPM + u, tt = e / 16, r = e % 16;
                    const float w =
                        __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][r], p.scale_log2, -m_w));
                    rs += w;
                    pf[2 * tt + r / 8][r % 8] = (_Float16)w;
                }
            }
        };
        if constexpr (T::PIPE) {
            if (!dead_next)
                weights_and_scores(std::true_type{});
            else
                weights_and_scores(std::false_type{});
        }
        l += rs;

        // O^T += V^T P^T
#pragma unroll
        for (int c = 0; c < 4; c++) {
#pragma unroll
            for (int dt = 0; dt < T::DT; dt++) {
                const char *a = vs_tile + voff[dt] + 16 * c * T::ROWB;
                const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) short4v *)TGA_LDS(a));
                const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) short4v *)TGA_LDS(a + 8 * T::ROWB));
                const half8 vf = __builtin_bit_cast(
                    half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[c], acc[dt], 0, 0, 0);
            }
        }
        if constexpr (T::PIPE) {
            if (j + 1 < nblk)
                mx_next = dead_next ? -INFINITY : tile_max(sn, j + 1);
        }
    };

    using J0 = std::integral_constant<int, 0>;
    using J1 = std::integral_constant<int, 1>;
    int j = 0;
    for (; j + T::U <= nblk; j += T::U) {
        step(J0{}, j);
        if constexpr (T::U == 2)
            step(J1{}, j + 1);
    }
    if (T::U == 2 && j < nblk)
        step(J0{}, j);

    // O = O^T / l, row by row; lse = (m + log2 l) ln 2
    const float lsum = l + __shfl_xor(l, 32);
    if (query < p.Lq) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        _Float16 *orow = p.O + b * p.os[0] + hq * p.os[1] + (int64_t)query * p.os[2];
#pragma unroll
        for (int dt = 0; dt < T::DT; dt++) {
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const half4 v = {(_Float16)(acc[dt][4 * g] * inv), (_Float16)(acc[dt][4 * g + 1] * inv),
                                 (_Float16)(acc[dt][4 * g + 2] * inv),
                                 (_Float16)(acc[dt][4 * g + 3] * inv)};
                *(half4 *)(orow + 32 * dt + 8 * g + 4 * h) = v;
            }
        }
        if (p.lse != nullptr && h == 0)
            p.lse[((int64_t)b * p.H + hq) * p.Lq + query] =
                lsum > 0.f ? (m + __builtin_amdgcn_logf(lsum)) * 0.6931471805599453f : -INFINITY;
    }
}

}  // namespace attn

hipError_t launch_attention(const AttentionArgs &a, hipStream_t s)
{
    attn::AttnParams p;
    p.Q = static_cast<const _Float16 *>(a.Q);
    p.K = static_cast<const _Float16 *>(a.K);
    p.V = static_cast<const _Float16 *>(a.V);
    p.O = static_cast<_Float16 *>(a.O);
    p.lse = a.lse;
    p.B = a.B;
    p.H = a.H;
    p.group = a.H / a.Hkv;
    p.Lq = a.Lq;
    p.Lk = a.Lk;
    for (int i = 0; i < 3; i++) {
        p.qs[i] = a.qs[i];
        p.ks[i] = a.ks[i];
        p.vs[i] = a.vs[i];
        p.os[i] = a.os[i];
    }
    p.k_bytes = a.k_bytes;
    p.v_bytes = a.v_bytes;
    // The kernel scales raw scores by this positive factor inside the
    // exponent, with -inf for masked keys.  A scale of magnitude below 2^-100
    // (zero included) makes every weight exp(scale (s_j - s_max)) round to
    // exactly 1 in fp32 for any fp16 scores: that case runs with Q read as
    // zeros and the factor log2(e), whose scores are exactly 0 -- the uniform
    // weights, computed exactly (a zero factor would turn -inf into NaN).
    const float mag = fabsf(a.scale);
    p.zero_q = mag < 0x1p-100f;
    p.scale_log2 = (p.zero_q ? 1.f : mag) * 1.4426950408889634f;
    p.negate_q = a.scale < 0.f;
    p.nqb = (a.Lq + attn::BQ - 1) / attn::BQ;
    p.causal = a.causal;
    const int64_t blocks = (int64_t)a.B * a.H * p.nqb;
    if (blocks <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)blocks), block(attn::THREADS);
    if (a.d == 64) {
        if (a.causal)
            hipLaunchKernelGGL((attn::attn_fwd<64, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((attn::attn_fwd<64, false>), grid, block, 0, s, p);
    } else if (a.d == 128) {
        if (a.causal)
            hipLaunchKernelGGL((attn::attn_fwd<128, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((attn::attn_fwd<128, false>), grid, block, 0, s, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tg
