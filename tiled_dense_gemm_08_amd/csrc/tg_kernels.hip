// tg_kernels.hip — gfx950 (MI355X, CDNA4) kernels of the tiled fp16 GEMM.
//
// The computation is the tiled matrix multiply of the TileLang pages: a grid of
// output tiles, a register-resident fp32 accumulator per tile, operand tiles
// staged through on-chip memory by a multi-stage software pipeline over K, a
// block-level matrix-multiply-accumulate, and an epilogue that writes the tile
// (lqnn.cn walkthrough, sections 2.1-2.2; codechina.net article, section 3.2),
// optionally fused with a per-column bias and ReLU (xdnf.cn article, section
// 4.2).  The pages' kernels target NVIDIA shared memory and warps; this file is
// written for CDNA4 instead:
//
//  * workgroups of 64-lane waves; each wave owns a TM x TN slab of the output
//    tile as 16x16 blocks of v_mfma_f32_16x16x32_f16 accumulators (4 fp32 per
//    lane per block);
//  * operands reach LDS either by 16-byte direct global->LDS DMA through
//    buffer descriptors (bounds give zeros for free), or through registers
//    with per-element bounds checks for operands of any alignment;
//  * a ring of STAGES LDS buffers over the K loop, one workgroup barrier per
//    K step, LDS-only fences so that prefetches stay in flight across it;
//  * XOR swizzles on the 16-byte chunk index of each LDS row, chosen so that
//    the fragment reads of a wave spread over all LDS banks (the pages use a
//    swizzle or row padding for the same purpose: pwwt.cn article, section
//    3.3; codechina.net article, section 4.1);
//  * A fragments come from ds_read_b128 on k-contiguous rows; B is row-major
//    (n-contiguous), and its fragments come from ds_read_b64_tr_b16, the
//    gfx950 LDS transpose read, so B is never transposed in memory;
//  * the MFMA is issued with the operands swapped (B fragment as the first
//    source) so that each lane ends with 4 consecutive columns of one output
//    row: 16-byte fp32 or 8-byte fp16 stores and a 16-byte bias load;
//  * workgroup ids are remapped so that each of the 8 XCDs (each with its own
//    L2) works on a contiguous, grouped band of output tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_kernels.h"

namespace tg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

#define TG_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Offset that lies beyond every buffer's num_records: a buffer load from it
// returns zeros.  Valid offsets are kept below it (operands < 2 GiB).
static constexpr uint32_t kOOB = 0x80000000u;

// gfx9 buffer resource word 3 (raw buffer, 32-bit data format).
static constexpr int kRsrcWord3 = 0x00020000;

// ---------------------------------------------------------------- barriers --
// Workgroup barrier that orders LDS only: outstanding global->LDS prefetches
// and global loads stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---------------------------------------------------------------- swizzles --
// A tile in LDS: BM rows of BK fp16 (k contiguous), 16-byte chunks XOR-
// swizzled by row.  A fragment read has 16 lanes on 16 consecutive rows at the
// same logical chunk; the swizzle sends them to 16 distinct 16-byte slots of
// any 256-byte window (and 8 consecutive rows to 8 slots of 128 bytes).
template <int BK>
__device__ __forceinline__ int swz_a(int row)
{
    if constexpr (BK == 64)
        return (row & 7) ^ ((row >> 3) & 1);
    else  // BK == 32: 4 chunks per 64-byte row
        return ((row >> 1) & 3) ^ ((row >> 3) & 1);
}

// B tile in LDS: BK rows of BN fp16 (n contiguous).  A transpose read has, per
// 16-lane group, 4 rows (k % 4 = 0..3) of 32 bytes, and the 4 groups sit on
// rows 8 apart; the swizzle (multiples of 2 chunks, so the 32-byte pairs stay
// whole) spreads rows {0..3, 8..11} over 8 distinct 32-byte slots.  It must
// stay below the BN/8 chunks of a row, so 64-wide tiles use only the k % 4 part.
template <int BN>
__device__ __forceinline__ int swz_b(int k)
{
    if constexpr (BN >= 128)
        return 2 * (k & 3) + 8 * ((k >> 3) & 1);
    else
        return 2 * (k & 3);
}

// ------------------------------------------------------------- tile order --
// Workgroup ids are dealt round-robin to the 8 XCDs; give each XCD a
// contiguous range of logical tiles, then walk tiles in groups of GROUP_M
// tile-rows so that concurrently running tiles share A rows and B columns.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int group_m,
                                            int &tm, int &tn)
{
    const int G = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int xcd = b & 7, slot = b >> 3;
    const int per = G >> 3, rem = G & 7;
    const int t = xcd * per + (xcd < rem ? xcd : rem) + slot;
    const int group_size = group_m * tiles_n;
    const int g = t / group_size;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int r = t - g * group_size;
    tm = first_m + r % gm;
    tn = r / gm;
}

// ---------------------------------------------------------------- configs --
template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WM_, WAVES_N = WN_;
    static constexpr int STAGES = STAGES_;
    static constexpr int WAVES = WM_ * WN_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TM = BM / WM_, TN = BN / WN_;     // wave tile
    static constexpr int MT = TM / 16, NT = TN / 16;       // MFMA blocks per wave
    static constexpr int KS = BK / 32;                     // MFMA k-steps per K step
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BK * BN * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    // global->LDS copy: each wave instruction moves 1 KiB (64 lanes x 16 B)
    static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;  // per thread per K step
    static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    static constexpr int A_ROWS_PER_LOAD = 1024 / (BK * 2);
    static constexpr int B_ROWS_PER_LOAD = 1024 / (BN * 2);
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0, "copy split");
    static_assert(BN * 2 <= 1024 && BN % 64 == 0, "BN");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// ------------------------------------------------------- fragment compute --
// One K step out of LDS stage `as` (A) / `bs` (B): KS MFMA k-steps of 32.
template <class C>
__device__ __forceinline__ void compute_stage(const char *as, const char *bs,
                                              const int (&a_off)[C::KS],
                                              const int (&b_off)[C::NT],
                                              float4v (&acc)[C::MT][C::NT])
{
#pragma unroll
    for (int ks = 0; ks < C::KS; ks++) {
        half8 af[C::MT];
        half8 bf[C::NT];
#pragma unroll
        for (int mt = 0; mt < C::MT; mt++)
            af[mt] = *(const half8 *)(as + a_off[ks] + mt * 16 * C::BK * 2);
#pragma unroll
        for (int nt = 0; nt < C::NT; nt++) {
            const char *p = bs + b_off[nt] + ks * 32 * C::BN * 2;
            short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v *)TG_LDS(p));
            short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4v *)TG_LDS(p + 4 * C::BN * 2));
            bf[nt] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int mt = 0; mt < C::MT; mt++)
#pragma unroll
            for (int nt = 0; nt < C::NT; nt++)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[nt], af[mt],
                                                                    acc[mt][nt], 0, 0, 0);
    }
}

// ---------------------------------------------------------------- epilogue --
// Lane l holds, for block (mt, nt), row (l % 16) and columns 4*(l/16) .. +3.
template <class C, typename OutT, bool BIAS>
__device__ __forceinline__ void epilogue(const Params &p, int m_base, int n_base,
                                         float4v (&acc)[C::MT][C::NT])
{
    const int lane = threadIdx.x & 63;
    const bool vec_ok = p.vec_store != 0;
#pragma unroll
    for (int nt = 0; nt < C::NT; nt++) {
        const int col = n_base + nt * 16 + 4 * (lane >> 4);
        float4v bv = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BIAS) {
            if (p.vec_bias && col + 3 < p.N) {
                bv = *(const float4v *)(p.bias + col);
            } else {
#pragma unroll
                for (int r = 0; r < 4; r++)
                    bv[r] = (col + r < p.N) ? p.bias[col + r] : 0.f;
            }
        }
#pragma unroll
        for (int mt = 0; mt < C::MT; mt++) {
            const int row = m_base + mt * 16 + (lane & 15);
            if (row >= p.M)
                continue;
            float4v v = acc[mt][nt];
            if constexpr (BIAS) {
#pragma unroll
                for (int r = 0; r < 4; r++)
                    v[r] = fmaxf(v[r] + bv[r], 0.f);
            }
            OutT *dst = (OutT *)p.C + (int64_t)row * p.ldc + col;
            if (vec_ok && col + 3 < p.N) {
                if constexpr (sizeof(OutT) == 4) {
                    *(float4v *)dst = v;
                } else {
                    half4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
                    *(half4 *)dst = h;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; r++)
                    if (col + r < p.N)
                        dst[r] = (OutT)v[r];
            }
        }
    }
}

// --------------------------------------------- per-lane LDS read offsets --
template <class C>
__device__ __forceinline__ void fragment_offsets(int wm, int wn, int (&a_off)[C::KS],
                                                 int (&b_off)[C::NT])
{
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;     // 16-lane group: which 8 k of the 32
    const int i = lane & 15;
#pragma unroll
    for (int ks = 0; ks < C::KS; ks++) {
        const int row = wm * C::TM + i;                  // + mt * 16 (swizzle-neutral)
        const int chunk = ks * 4 + g;
        a_off[ks] = row * C::BK * 2 + ((chunk ^ swz_a<C::BK>(row)) * 16);
    }
    // transpose read: lane 16g + 4e + q supplies row k = 8g + e (+4 for the
    // second read, + 32 per MFMA k-step), columns 4q .. 4q+3 of the 16-wide
    // slice; the hardware hands lane 16g + j the column j of those 4 rows.
    const int e = i >> 2, q = i & 3;
    const int k = 8 * g + e;
#pragma unroll
    for (int nt = 0; nt < C::NT; nt++) {
        const int col = wn * C::TN + nt * 16 + 4 * q;
        const int chunk = col >> 3;
        b_off[nt] = k * C::BN * 2 + ((chunk ^ swz_b<C::BN>(k)) * 16) + (col & 7) * 2;
    }
}

// ============================================================================
// Direct path: 16-byte global->LDS DMA.  Requires 16-byte aligned A and B,
// lda % 8 == 0, ldb % 8 == 0, K % 8 == 0 and N % 8 == 0 so that every 16-byte
// chunk is either entirely inside the matrix or entirely outside it.
// ============================================================================
// 16-byte global->LDS DMA: lane i's 16 bytes from buffer offset `voff` land
// at LDS address `lds` + 16 i.  Written as inline assembly so that the
// compiler does not treat every later LDS read as dependent on the copy (it
// would wait for all outstanding copies before each one); the kernel waits on
// vmcnt itself, before the barrier that publishes a stage.  M0 is written here
// and nowhere else in these kernels.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)p;
}

template <class C>
struct DirectLoader {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t a_base[C::A_LOADS];   // byte offset at k0 = 0, or kOOB
    uint32_t b_base[C::B_LOADS];
    int a_kchunk[C::A_LOADS];      // logical k-chunk of this lane's A load
    int b_krow[C::B_LOADS];        // k row (within the tile) of this lane's B load
    uint32_t a_step, b_step;       // bytes per K step

    __device__ __forceinline__ void init(const Params &p, int m0, int n0)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        ra = __builtin_amdgcn_make_buffer_rsrc((void *)p.A, 0, p.a_bytes, kRsrcWord3);
        rb = __builtin_amdgcn_make_buffer_rsrc((void *)p.B, 0, p.b_bytes, kRsrcWord3);
#pragma unroll
        for (int t = 0; t < C::A_LOADS; t++) {
            const int inst = wave * C::A_LOADS + t;
            const int row = inst * C::A_ROWS_PER_LOAD + lane / (C::BK / 8);
            const int phys = lane % (C::BK / 8);
            const int chunk = phys ^ swz_a<C::BK>(row);
            a_kchunk[t] = chunk;
            const int gm = m0 + row;
            a_base[t] = (gm < p.M) ? (uint32_t)(((int64_t)gm * p.lda + chunk * 8) * 2) : kOOB;
        }
#pragma unroll
        for (int t = 0; t < C::B_LOADS; t++) {
            const int inst = wave * C::B_LOADS + t;
            const int k = inst * C::B_ROWS_PER_LOAD + lane / (C::BN / 8);
            const int phys = lane % (C::BN / 8);
            const int chunk = phys ^ swz_b<C::BN>(k);
            b_krow[t] = k;
            const int gn = n0 + chunk * 8;
            b_base[t] = (gn < p.N) ? (uint32_t)(((int64_t)k * p.ldb + gn) * 2) : kOOB;
        }
        a_step = C::BK * 2;
        b_step = (uint32_t)(C::BK * p.ldb * 2);
    }

    // Issue the copies of K step kt into LDS stage base `dst`.
    __device__ __forceinline__ void issue(const Params &p, int kt, char *dst, bool tail)
    {
        const int wave = threadIdx.x >> 6;
        const uint32_t dst_lds = lds_addr(dst);
        const int k0 = kt * C::BK;
#pragma unroll
        for (int t = 0; t < C::A_LOADS; t++) {
            uint32_t off = a_base[t] + (uint32_t)kt * a_step;
            if (tail && k0 + a_kchunk[t] * 8 >= p.K)
                off = kOOB;
            dma16(ra, off, __builtin_amdgcn_readfirstlane(dst_lds + (wave * C::A_LOADS + t) * 1024));
        }
#pragma unroll
        for (int t = 0; t < C::B_LOADS; t++) {
            uint32_t off = b_base[t] + (uint32_t)kt * b_step;
            if (tail && k0 + b_krow[t] >= p.K)
                off = kOOB;
            dma16(rb, off,
                  __builtin_amdgcn_readfirstlane(dst_lds + C::A_BYTES + (wave * C::B_LOADS + t) * 1024));
        }
    }
};

template <class C, typename OutT, bool BIAS>
__global__ void __launch_bounds__(C::THREADS, 1) gemm_direct(Params p)
{
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
    int tm, tn;
    tile_coords(p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    float4v acc[C::MT][C::NT];
#pragma unroll
    for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int j = 0; j < C::NT; j++)
            acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

    int a_off[C::KS], b_off[C::NT];
    fragment_offsets<C>(wm, wn, a_off, b_off);

    DirectLoader<C> ld;
    ld.init(p, m0, n0);
    const int nk = (p.K + C::BK - 1) / C::BK;
    const bool ragged_k = (p.K % C::BK) != 0;

#pragma unroll
    for (int s = 0; s < C::STAGES - 1; s++)
        if (s < nk)
            ld.issue(p, s, smem + s * C::STAGE_BYTES, ragged_k && s == nk - 1);

    for (int kt = 0; kt < nk; kt++) {
        // this lane's copies of step kt are done once at most the copies of
        // the STAGES-2 later steps are still outstanding
        if (kt + C::STAGES - 2 < nk)
            wait_vmcnt<(C::STAGES - 2) * C::LOADS>();
        else
            wait_vmcnt<0>();
        lds_barrier();   // everyone's copies of step kt landed; stage (kt-1) is free
        const int kn = kt + C::STAGES - 1;
        if (kn < nk)
            ld.issue(p, kn, smem + (kn % C::STAGES) * C::STAGE_BYTES, ragged_k && kn == nk - 1);
        const char *as = smem + (kt % C::STAGES) * C::STAGE_BYTES;
        compute_stage<C>(as, as + C::A_BYTES, a_off, b_off, acc);
    }
    epilogue<C, OutT, BIAS>(p, m0 + wm * C::TM, n0 + wn * C::TN, acc);
}

// ============================================================================
// General path: register-staged copies with per-element bounds; any pointer
// alignment (2-byte) and any leading dimensions.  Same LDS layout and compute.
// ============================================================================
template <class C>
struct StagedLoader {
    half8 ra[C::A_LOADS];
    half8 rb[C::B_LOADS];

    __device__ __forceinline__ void load(const Params &p, int m0, int n0, int kt)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int k0 = kt * C::BK;
        const _Float16 *A = p.A, *B = p.B;
#pragma unroll
        for (int t = 0; t < C::A_LOADS; t++) {
            const int inst = wave * C::A_LOADS + t;
            const int row = inst * C::A_ROWS_PER_LOAD + lane / (C::BK / 8);
            const int phys = lane % (C::BK / 8);
            const int kc = k0 + (phys ^ swz_a<C::BK>(row)) * 8;
            const int gm = m0 + row;
            half8 v;
            if (gm < p.M) {
                const _Float16 *src = A + (int64_t)gm * p.lda + kc;
                if (p.a_vec && kc + 7 < p.K) {
                    v = *(const half8 *)src;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        v[e] = (kc + e < p.K) ? src[e] : (_Float16)0.f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    v[e] = (_Float16)0.f;
            }
            ra[t] = v;
        }
#pragma unroll
        for (int t = 0; t < C::B_LOADS; t++) {
            const int inst = wave * C::B_LOADS + t;
            const int k = inst * C::B_ROWS_PER_LOAD + lane / (C::BN / 8);
            const int phys = lane % (C::BN / 8);
            const int gn = n0 + (phys ^ swz_b<C::BN>(k)) * 8;
            const int gk = k0 + k;
            half8 v;
            if (gk < p.K) {
                const _Float16 *src = B + (int64_t)gk * p.ldb + gn;
                if (p.b_vec && gn + 7 < p.N) {
                    v = *(const half8 *)src;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        v[e] = (gn + e < p.N) ? src[e] : (_Float16)0.f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    v[e] = (_Float16)0.f;
            }
            rb[t] = v;
        }
    }

    __device__ __forceinline__ void store(char *dst)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int t = 0; t < C::A_LOADS; t++)
            *(half8 *)(dst + (wave * C::A_LOADS + t) * 1024 + lane * 16) = ra[t];
#pragma unroll
        for (int t = 0; t < C::B_LOADS; t++)
            *(half8 *)(dst + C::A_BYTES + (wave * C::B_LOADS + t) * 1024 + lane * 16) = rb[t];
    }
};

template <class C, typename OutT, bool BIAS>
__global__ void __launch_bounds__(C::THREADS, 1) gemm_staged(Params p)
{
    static_assert(C::STAGES == 2, "the register-staged path double-buffers LDS");
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
    int tm, tn;
    tile_coords(p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    float4v acc[C::MT][C::NT];
#pragma unroll
    for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int j = 0; j < C::NT; j++)
            acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

    int a_off[C::KS], b_off[C::NT];
    fragment_offsets<C>(wm, wn, a_off, b_off);

    const int nk = (p.K + C::BK - 1) / C::BK;
    StagedLoader<C> ld;
    if (nk > 0) {
        ld.load(p, m0, n0, 0);
        ld.store(smem);
    }
    lds_barrier();
    for (int kt = 0; kt < nk; kt++) {
        if (kt + 1 < nk)
            ld.load(p, m0, n0, kt + 1);
        const char *as = smem + (kt & 1) * C::STAGE_BYTES;
        compute_stage<C>(as, as + C::A_BYTES, a_off, b_off, acc);
        if (kt + 1 < nk)
            ld.store(smem + ((kt + 1) & 1) * C::STAGE_BYTES);
        lds_barrier();
    }
    epilogue<C, OutT, BIAS>(p, m0 + wm * C::TM, n0 + wn * C::TN, acc);
}

// ------------------------------------------------------------ instances --
template <class C, bool DIRECT>
hipError_t launch_cfg(const Params &p, bool f16_out, bool bias, hipStream_t s)
{
    const dim3 grid(p.tiles_m * p.tiles_n), block(C::THREADS);
#define TG_GO(KERNEL, OUT, B)                                                        \
    do {                                                                             \
        hipLaunchKernelGGL((KERNEL<C, OUT, B>), grid, block, 0, s, p);               \
        return hipGetLastError();                                                    \
    } while (0)
    if constexpr (DIRECT) {
        if (f16_out) { if (bias) TG_GO(gemm_direct, _Float16, true); else TG_GO(gemm_direct, _Float16, false); }
        else { if (bias) TG_GO(gemm_direct, float, true); else TG_GO(gemm_direct, float, false); }
    } else {
        if (f16_out) { if (bias) TG_GO(gemm_staged, _Float16, true); else TG_GO(gemm_staged, _Float16, false); }
        else { if (bias) TG_GO(gemm_staged, float, true); else TG_GO(gemm_staged, float, false); }
    }
#undef TG_GO
}

// Explicit instantiation: both compile passes see every kernel instance.
#define TG_CONFIG_ROW(ID, BM, BN, BK, WM, WN, ST, DIRECT)                            \
    template hipError_t launch_cfg<Cfg<BM, BN, BK, WM, WN, ST>, DIRECT>(             \
        const Params &, bool, bool, hipStream_t);
#include "tg_config_list.inc"
#undef TG_CONFIG_ROW

// The launch table is host data (the device pass would otherwise turn the
// const array into device constant memory).
#if !defined(__HIP_DEVICE_COMPILE__)
#define TG_CONFIG_ROW(ID, BM, BN, BK, WM, WN, ST, DIRECT)                            \
    {ID, BM, BN, BK, ST, WM, WN, DIRECT, Cfg<BM, BN, BK, WM, WN, ST>::LDS_BYTES,       \
     (DIRECT ? "direct_" #BM "x" #BN "x" #BK "_s" #ST "_w" #WM "x" #WN                \
             : "staged_" #BM "x" #BN "x" #BK "_s" #ST "_w" #WM "x" #WN),             \
     &launch_cfg<Cfg<BM, BN, BK, WM, WN, ST>, DIRECT>},

const KernelConfig kConfigs[] = {
#include "tg_config_list.inc"
};
const int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
#endif

}  // namespace tg
