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
//    tile as MI x MI blocks of MFMA accumulators, MI = 16
//    (v_mfma_f32_16x16x32_f16, 4 fp32 per lane per block) or MI = 32
//    (v_mfma_f32_32x32x16_f16, 16 fp32 per lane per block);
//  * operands reach LDS either by 16-byte direct global->LDS DMA through
//    buffer descriptors (bounds give zeros for free), or through registers
//    with per-element bounds checks for operands of any alignment;
//  * a ring of STAGES LDS buffers over the K loop, one workgroup barrier per
//    K step, LDS-only fences so that prefetches stay in flight across it;
//  * XOR swizzles on the 16-byte chunk index of each LDS row, chosen so that
//    the fragment reads of a wave spread over the LDS banks (the pages use a
//    swizzle or row padding for the same purpose: pwwt.cn article, section
//    3.3; codechina.net article, section 4.1);
//  * A fragments come from ds_read_b128 on k-contiguous rows; B is row-major
//    (n-contiguous), and its fragments come from ds_read_b64_tr_b16, the
//    gfx950 LDS transpose read, so B is never transposed in memory;
//  * the MFMA is issued with the operands swapped (B fragment as the first
//    source) so that each lane ends with runs of 4 consecutive columns of one
//    output row: 16-byte fp32 or 8-byte fp16 stores and a 16-byte bias load;
//  * workgroup ids are remapped so that each of the 8 XCDs (each with its own
//    L2) works on a contiguous, grouped band of output tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "tg_kernels.h"

namespace tg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));

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
// swizzled by row.  A fragment read has MI lanes on MI consecutive rows at
// the same logical chunk.  With 128-byte rows, XOR by (row & 7) reads at the
// full ds_read_b128 rate on gfx950 (measured: about 200 B/clk/CU, against
// about 60 without a swizzle).  64-byte rows (BK = 32) use a 2-bit analogue.
// Both are unchanged by row += 16, so one per-lane offset serves every block.
template <int BK>
__device__ __forceinline__ int swz_a(int row)
{
    if constexpr (BK == 64)
        return row & 7;
    else
        return (row >> 1) & 3;
}

// B tile in LDS: BK rows of BN fp16 (n contiguous).  A transpose read has, per
// 16-lane group, 4 rows (k % 4 = 0..3) of 32 bytes, and groups sit on rows 8
// apart; the swizzle (multiples of 2 chunks, so the 32-byte pairs stay whole)
// spreads rows {0..3, 8..11} over 8 distinct 32-byte slots.  It must stay
// below the BN/8 chunks of a row, so 64-wide tiles use only the k % 4 part.
// It is unchanged by k += 4 and k += 16.
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
// contiguous range of logical tiles, then walk tiles in groups of group_m
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
template <int MI> struct AccT;
template <> struct AccT<16> { typedef float4v type; };
template <> struct AccT<32> { typedef float16v type; };

template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int MI_, int SCHED_>
struct Cfg {
    static constexpr int SCHED = SCHED_;   // copy issue: 0 burst after the barrier, 1 spread
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WM_, WAVES_N = WN_;
    static constexpr int STAGES = STAGES_;
    static constexpr int MI = MI_;                         // MFMA block edge
    static constexpr int KI = 512 / MI;                    // k per MFMA: 32 or 16
    static constexpr int ACC = MI * MI / 64;               // fp32 per lane per block
    static constexpr int WAVES = WM_ * WN_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TM = BM / WM_, TN = BN / WN_;     // wave tile
    static constexpr int MT = TM / MI, NT = TN / MI;       // MFMA blocks per wave
    static constexpr int KS = BK / KI;                     // MFMA k-steps per K step
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
    typedef typename AccT<MI>::type acc_t;
    static_assert(MI == 16 || MI == 32, "MI");
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(TM % MI == 0 && TN % MI == 0, "wave tile");
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0, "copy split");
    static_assert(BN * 2 <= 1024 && BN % 64 == 0, "BN");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// ------------------------------------------------------------- fragments --
// Per-lane LDS byte offsets of the fragment reads (stage-relative).
//  A (MFMA second source): lane l holds row l % MI, k = 8 (l / MI) .. +7 of
//    the k-step: one ds_read_b128.  a_off[ks] + mt * MI * BK * 2 for block mt.
//  B (MFMA first source): lane l holds column l % MI, the same 8 k.  Two
//    transpose reads of 4 k each: lane L = 16 G + 4 e + q reads row
//    k = 8 (L / MI) + e (+4 for the second read, + KI per k-step) at columns
//    16 ((L % MI) / 16) + 4 q .. +3 of the block; the hardware hands lane
//    16 G + j the 4 rows' column j.  b_off[nt] for block nt.
template <class C>
__device__ __forceinline__ void fragment_offsets(int wm, int wn, int (&a_off)[C::KS],
                                                 int (&b_off)[C::NT])
{
    const int lane = threadIdx.x & 63;
    const int kgroup = lane / C::MI;
#pragma unroll
    for (int ks = 0; ks < C::KS; ks++) {
        const int row = wm * C::TM + lane % C::MI;
        const int chunk = ks * (C::KI / 8) + kgroup;
        a_off[ks] = row * C::BK * 2 + ((chunk ^ swz_a<C::BK>(row)) * 16);
    }
    const int i = lane & 15;
    const int e = i >> 2, q = i & 3;
    const int k = 8 * kgroup + e;
    const int sub = (lane % C::MI) >> 4;
#pragma unroll
    for (int nt = 0; nt < C::NT; nt++) {
        const int col = wn * C::TN + nt * C::MI + sub * 16 + 4 * q;
        b_off[nt] = k * C::BN * 2 + (((col >> 3) ^ swz_b<C::BN>(k)) * 16) + (col & 7) * 2;
    }
}

template <class C>
__device__ __forceinline__ void read_frags(const char *as, const char *bs, int ks,
                                           const int (&a_off)[C::KS], const int (&b_off)[C::NT],
                                           half8 (&fa)[C::MT], half8 (&fb)[C::NT])
{
#pragma unroll
    for (int nt = 0; nt < C::NT; nt++) {
        const char *q = bs + b_off[nt] + ks * C::KI * C::BN * 2;
        short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v *)TG_LDS(q));
        short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v *)TG_LDS(q + 4 * C::BN * 2));
        fb[nt] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int mt = 0; mt < C::MT; mt++)
        fa[mt] = *(const half8 *)(as + a_off[ks] + mt * C::MI * C::BK * 2);
}

template <class C>
__device__ __forceinline__ typename C::acc_t mfma(half8 b, half8 a, typename C::acc_t c)
{
    if constexpr (C::MI == 16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0);
}

template <class C, int LO, int HI>
__device__ __forceinline__ void mfma_range(const half8 (&fa)[C::MT], const half8 (&fb)[C::NT],
                                           typename C::acc_t (&acc)[C::MT][C::NT])
{
#pragma unroll
    for (int i = LO; i < HI; i++) {
        const int mt = i / C::NT, nt = i % C::NT;
        acc[mt][nt] = mfma<C>(fb[nt], fa[mt], acc[mt][nt]);
    }
}

// ---------------------------------------------------------------- epilogue --
// After the operand swap, lane l holds for block (mt, nt) row l % MI of the
// block and, for each run r4 < ACC / 4, the 4 consecutive columns
// 8 r4 + 4 (l / 32) .. +3 (MI = 32) or 4 (l / 16) .. +3 (MI = 16).
template <class C>
__device__ __forceinline__ int run_col(int nt, int run)
{
    const int lane = threadIdx.x & 63;
    return nt * C::MI + 8 * run + 4 * (lane / C::MI);
}

// Bias for 4 consecutive columns starting at col (zeros past N).
__device__ __forceinline__ float4v load_bias4(const Params &p, int col)
{
    float4v bv = {0.f, 0.f, 0.f, 0.f};
    if (p.vec_bias && col + 3 < p.N) {
        bv = *(const float4v *)(p.bias + col);
    } else {
#pragma unroll
        for (int r = 0; r < 4; r++)
            bv[r] = (col + r < p.N) ? p.bias[col + r] : 0.f;
    }
    return bv;
}

template <class C, bool BIAS>
__device__ __forceinline__ float4v epi_value(const typename C::acc_t &a, int run, float4v bv)
{
    float4v v;
#pragma unroll
    for (int r = 0; r < 4; r++)
        v[r] = a[4 * run + r];
    if constexpr (BIAS) {
#pragma unroll
        for (int r = 0; r < 4; r++)
            v[r] = fmaxf(v[r] + bv[r], 0.f);
    }
    return v;
}

// Direct epilogue: each lane stores its 4-column runs straight to C.  Used when
// C's rows do not allow 16-byte stores (unaligned base or leading dimension).
template <class C, typename OutT, bool BIAS>
__device__ __forceinline__ void epilogue_direct(const Params &p, int m_base, int n_base,
                                                typename C::acc_t (&acc)[C::MT][C::NT])
{
    const int lane = threadIdx.x & 63;
    const bool vec_ok = p.vec_store != 0;
    constexpr int RUNS = C::ACC / 4;
#pragma unroll
    for (int nt = 0; nt < C::NT; nt++) {
#pragma unroll
        for (int run = 0; run < RUNS; run++) {
            const int col = n_base + run_col<C>(nt, run);
            float4v bv = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BIAS)
                bv = load_bias4(p, col);
#pragma unroll
            for (int mt = 0; mt < C::MT; mt++) {
                const int row = m_base + mt * C::MI + lane % C::MI;
                if (row >= p.M)
                    continue;
                const float4v v = epi_value<C, BIAS>(acc[mt][nt], run, bv);
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
}

// Largest power-of-two fraction of the wave tile's rows that fits the budget.
constexpr int pass_rows(int tm, int fit)
{
    int r = tm;
    while (r > fit && r > 1)
        r /= 2;
    return r;
}

// Staged epilogue: the wave writes its converted tile, PR rows at a time, into
// a private LDS region in row-major order (rows padded by 16 bytes so that the
// 32 rows one MFMA block spans spread over the banks), then reads it back so
// that consecutive lanes hold consecutive 16-byte chunks of a row, and stores
// those: every store instruction writes whole 128-byte lines of C instead of
// 16 bytes in each of 32 rows.  The caller has made the workgroup's LDS free
// (no copy in flight, every wave past its last fragment read).
template <class C, typename OutT, bool BIAS>
__device__ __forceinline__ void epilogue_lds(const Params &p, char *smem, int m_base, int n_base,
                                             typename C::acc_t (&acc)[C::MT][C::NT])
{
    constexpr int ES = sizeof(OutT);
    constexpr int ROWB = C::TN * ES + 16;                  // padded LDS row
    constexpr int REGION = (C::LDS_BYTES / C::WAVES) & ~15;
    constexpr int PR = pass_rows(C::TM, REGION / ROWB);   // rows per pass
    static_assert(PR >= C::MI && C::TM % PR == 0, "epilogue staging region");
    constexpr int CPR = C::TN * ES / 16;                   // 16-byte chunks per row
    static_assert((PR * CPR) % 64 == 0, "whole read-back instructions");
    constexpr int RUNS = C::ACC / 4;
    constexpr int MT_PASS = PR / C::MI;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    char *region = smem + wave * REGION;

#pragma unroll
    for (int pass = 0; pass < C::TM / PR; pass++) {
        // registers -> LDS (row-major, padded rows)
#pragma unroll
        for (int nt = 0; nt < C::NT; nt++)
#pragma unroll
            for (int run = 0; run < RUNS; run++) {
                float4v bv = {0.f, 0.f, 0.f, 0.f};
                if constexpr (BIAS)
                    bv = load_bias4(p, n_base + run_col<C>(nt, run));
#pragma unroll
                for (int i = 0; i < MT_PASS; i++) {
                    const int mt = pass * MT_PASS + i;
                    const int row = i * C::MI + lane % C::MI;
                    const float4v v = epi_value<C, BIAS>(acc[mt][nt], run, bv);
                    char *dst = region + row * ROWB + run_col<C>(nt, run) * ES;
                    if constexpr (ES == 4) {
                        *(float4v *)dst = v;
                    } else {
                        half4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
                        *(half4 *)dst = h;
                    }
                }
        }
        // LDS -> C, 16 bytes per lane, consecutive lanes along a row.  A wave's
        // LDS accesses complete in order, so no barrier is needed: the region
        // is private to this wave.
#pragma unroll
        for (int it = 0; it < PR * CPR / 64; it++) {
            const int q = it * 64 + lane;
            const int r = q / CPR, cc = q % CPR;
            const float4v v = *(const float4v *)(region + r * ROWB + cc * 16);
            const int row = m_base + pass * PR + r;
            const int col = n_base + cc * (16 / ES);
            if (row < p.M) {
                OutT *dst = (OutT *)p.C + (int64_t)row * p.ldc + col;
                if (col + 16 / ES <= p.N) {
                    *(float4v *)dst = v;
                } else {
                    const OutT *e = (const OutT *)&v;
#pragma unroll
                    for (int j = 0; j < 16 / ES; j++)
                        if (col + j < p.N)
                            dst[j] = e[j];
                }
            }
        }
    }
}

template <class C, typename OutT, bool BIAS>
__device__ __forceinline__ void epilogue(const Params &p, char *smem, int m_base, int n_base,
                                         typename C::acc_t (&acc)[C::MT][C::NT])
{
    if (p.line_store)
        epilogue_lds<C, OutT, BIAS>(p, smem, m_base, n_base, acc);
    else
        epilogue_direct<C, OutT, BIAS>(p, m_base, n_base, acc);
}

// ============================================================================
// Direct copies: 16-byte global->LDS DMA.  Requires 16-byte aligned A and B,
// lda % 8 == 0, ldb % 8 == 0, K % 8 == 0 and N % 8 == 0 so that every 16-byte
// chunk is either entirely inside the matrix or entirely outside it.
// ============================================================================
// Lane i's 16 bytes from buffer offset `voff` land at LDS address lds + 16 i.
// Written as inline assembly so that the compiler does not treat every later
// LDS read as dependent on the copy (it would wait for all outstanding copies
// before each one); the kernels wait on vmcnt themselves, before the barrier
// that publishes a stage.  M0 is written here and nowhere else in these
// kernels (the build checks the device assembly for that).  A scalar write of
// M0 needs one wait state before a load that uses it as the LDS address.
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

// Wave w's copy instruction t of a K step fills LDS bytes [1 KiB * (w *
// LOADS + t), +1 KiB) of the A (or B) tile: A_ROWS_PER_LOAD rows of the A tile
// (lane -> row lane / (BK/8), physical chunk lane % (BK/8)), or
// B_ROWS_PER_LOAD k-rows of the B tile.  The swizzle is applied on the global
// side: each lane fetches the logical chunk that belongs at its physical slot.
//
// The K position is carried by the buffer descriptors, not by the lane
// offsets: for K step kt the A descriptor starts at A + kt*BK with its range
// shortened by as much, and likewise for B, so the lane offsets are constants
// of the tile and a K step costs a few scalar instructions.  The range check
// of the descriptor gives zeros for the rows of A past M and the rows of B
// past K (the host guarantees that those offsets do not wrap 32 bits);
// columns of B past N and the columns of A past K in the last K step lie
// inside the buffer and are pushed out of range explicitly.  Steps at or past
// nk get a zero-length descriptor: every lane reads zeros without touching
// memory, so each K step keeps the same number of outstanding copies.
template <class C>
struct DirectLoader {
    // Per-instruction lane offsets are kept in registers when there are few
    // of them; otherwise they are rebuilt at issue from lane constants.
    static constexpr bool KEEP = C::LOADS <= 8;
    uint32_t voff[KEEP ? C::LOADS : 1];
    uint32_t a_lane;   // A: byte offset of this lane's chunk in instruction 0
    int a_kc8;         // A: logical k offset of this lane's chunk in the tile
    int b_row, b_phys; // B: k-row within an instruction; physical chunk
    uint32_t lds0;     // LDS byte address of the workgroup's buffer

    __device__ __forceinline__ uint32_t a_off(const Params &p, int t) const
    {
        const int inst = (threadIdx.x >> 6) * C::A_LOADS + t;
        return a_lane + (uint32_t)(inst * C::A_ROWS_PER_LOAD) * (uint32_t)p.lda * 2u;
    }

    __device__ __forceinline__ uint32_t b_off(const Params &p, int t, int n0) const
    {
        const int inst = (threadIdx.x >> 6) * C::B_LOADS + t;
        const int k = inst * C::B_ROWS_PER_LOAD + b_row;
        const int col = n0 + (b_phys ^ swz_b<C::BN>(k)) * 8;
        return col < p.N ? ((uint32_t)k * (uint32_t)p.ldb + (uint32_t)col) * 2u : kOOB;
    }

    __device__ __forceinline__ void init(const Params &p, const char *smem, int m0, int n0)
    {
        const int lane = threadIdx.x & 63;
        const int a_row = lane / (C::BK / 8);
        // the A swizzle depends on row % A_ROWS_PER_LOAD only (8 or 16 rows)
        a_kc8 = ((lane % (C::BK / 8)) ^ swz_a<C::BK>(a_row)) * 8;
        a_lane = (uint32_t)(((int64_t)(m0 + a_row) * p.lda + a_kc8) * 2);
        b_row = lane / (C::BN / 8);
        b_phys = lane % (C::BN / 8);
        lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        if constexpr (KEEP) {
#pragma unroll
            for (int t = 0; t < C::A_LOADS; t++)
                voff[t] = a_off(p, t);
#pragma unroll
            for (int t = 0; t < C::B_LOADS; t++)
                voff[C::A_LOADS + t] = b_off(p, t, n0);
        }
    }

    // Issue copy instruction T (A copies first, then B) of K step kt into
    // LDS stage S.
    template <int S, int T>
    __device__ __forceinline__ void issue_one(const Params &p, int kt, int nk, int n0)
    {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const bool valid = kt < nk;
        const int k0 = kt * C::BK;
        if constexpr (T < C::A_LOADS) {
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.A + k0), 0, valid ? (int)(p.a_bytes - (uint32_t)k0 * 2u) : 0,
                kRsrcWord3);
            // K tail: this lane's A chunk lies past K (inside the row's padding
            // or the next row), so it is pushed out of range
            const bool a_dead = (kt == nk - 1) && (a_kc8 >= p.K - k0);
            const uint32_t o = KEEP ? voff[T] : a_off(p, T);
            dma16(ra, a_dead ? kOOB : o,
                  lds0 + S * C::A_BYTES + (wave * C::A_LOADS + T) * 1024);
        } else {
            constexpr int t = T - C::A_LOADS;
            const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.B + (int64_t)k0 * p.ldb), 0,
                valid ? (int)(p.b_bytes - (uint32_t)k0 * (uint32_t)p.ldb * 2u) : 0, kRsrcWord3);
            const uint32_t o = KEEP ? voff[T] : b_off(p, t, n0);
            dma16(rb, o,
                  lds0 + C::STAGES * C::A_BYTES + S * C::B_BYTES + (wave * C::B_LOADS + t) * 1024);
        }
    }

    // Copy instructions [T0, T1) of K step kt into LDS stage S.
    template <int S, int T0 = 0, int T1 = C::LOADS>
    __device__ __forceinline__ void issue(const Params &p, int kt, int nk, int n0)
    {
        if constexpr (T0 < T1) {
            issue_one<S, T0>(p, kt, nk, n0);
            issue<S, T0 + 1, T1>(p, kt, nk, n0);
        }
    }
};

// ============================================================================
// Pipelined direct kernel.  LDS holds STAGES A tiles followed by STAGES B
// tiles, so every fragment read of a stage is a lane base register plus an
// immediate offset.  The K loop is unrolled by STAGES K steps (stage indices
// are compile-time constants) and software-pipelined at MFMA k-step
// granularity:
//  * fragments are double-buffered in registers: while the MFMAs of k-step u
//    run, the LDS reads for k-step u+1 are in flight;
//  * the workgroup barrier that publishes K step kt+1 sits in the middle of
//    the last k-step of K step kt: half of its MFMAs are issued before the
//    barrier and half after, covering the barrier and the first fragment
//    reads of step kt+1;
//  * right after that barrier the copy of step kt+STAGES is issued into the
//    stage that step kt just vacated, so STAGES-1 K steps of compute cover
//    each copy's latency; copies past the end are zero-reading dummies, which
//    keeps the outstanding-copy count (and so the vmcnt wait) constant.
// The K-step count is padded to a multiple of STAGES with all-zero steps.
// ============================================================================
template <int N, int R>
__device__ __forceinline__ void sched_interleave_reads()
{
    if constexpr (N > 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, R, 0);   // then R MFMAs
        sched_interleave_reads<N - 1, R>();
    }
}

template <class C>
struct PipeState {
    int a_off[C::KS], b_off[C::NT];
    half8 fa[2][C::MT], fb[2][C::NT];
    typename C::acc_t acc[C::MT][C::NT];
};

template <class C, int S>
__device__ __forceinline__ const char *a_stage(const char *smem)
{
    return smem + S * C::A_BYTES;
}

template <class C, int S>
__device__ __forceinline__ const char *b_stage(const char *smem)
{
    return smem + C::STAGES * C::A_BYTES + S * C::B_BYTES;
}

// Spread copy schedule (SCHED = 1).  The barrier in the last k-step of K step
// S frees stage S; the copies that refill it (K step kt0 + S + STAGES) are
// issued one at a time between the MFMAs that follow, up to the next barrier
// (the "window" of stage S), instead of in one burst: in-order issue would
// otherwise hold every later MFMA behind copies waiting for the vector memory
// pipeline.  With two stages the next barrier waits for these very copies,
// so they are packed into the first half of the window.  Window positions
// count MFMAs from the barrier; a window that starts in the last k-step of a
// loop body ends in the next body (window -1 of that body).
template <class C>
struct Spread {
    static constexpr int NMF = C::MT * C::NT;
    static constexpr int H = NMF / 2;
    static constexpr int SPAN = C::STAGES == 2 ? C::KS * NMF / 2 : C::KS * NMF;
    static constexpr int pos(int t) { return t * SPAN / C::LOADS; }
};

// MFMA I of the current k-step, then the copies of window W whose position is
// OFF (window W refills stage (W + STAGES) % STAGES with K step kt0+W+STAGES).
template <class C, int W, int OFF, int T = 0>
__device__ __forceinline__ void window_copies(const Params &p, DirectLoader<C> &ld, int kt0, int nk,
                                              int n0)
{
    if constexpr (T < C::LOADS) {
        if constexpr (Spread<C>::pos(T) == OFF) {
            __builtin_amdgcn_sched_barrier(0);
            ld.template issue_one<(W + C::STAGES) % C::STAGES, T>(p, kt0 + W + C::STAGES, nk, n0);
            __builtin_amdgcn_sched_barrier(0);
        }
        window_copies<C, W, OFF, T + 1>(p, ld, kt0, nk, n0);
    }
}

// MFMAs [I, HI) of the k-step; MFMA I sits at position OFF of window W.
template <class C, int W, int OFF, int I, int HI>
__device__ __forceinline__ void mfma_window(const Params &p, DirectLoader<C> &ld, int kt0, int nk,
                                            int n0, const half8 (&fa)[C::MT],
                                            const half8 (&fb)[C::NT],
                                            typename C::acc_t (&acc)[C::MT][C::NT])
{
    if constexpr (I < HI) {
        constexpr int mt = I / C::NT, nt = I % C::NT;
        acc[mt][nt] = mfma<C>(fb[nt], fa[mt], acc[mt][nt]);
        window_copies<C, W, OFF>(p, ld, kt0, nk, n0);
        mfma_window<C, W, OFF + 1, I + 1, HI>(p, ld, kt0, nk, n0, fa, fb, acc);
    }
}

// k-step U (0 .. STAGES*KS-1) of a loop body; FINAL: the body that ends the
// K loop (no barrier, reads or copies after its last k-step).
template <class C, int U, bool FINAL>
__device__ __forceinline__ void pipe_kstep(const Params &p, DirectLoader<C> &ld, const char *smem,
                                           int kt0, int nk, int n0, PipeState<C> &st)
{
    constexpr int S = U / C::KS, ks = U % C::KS, P = U % 2;
    constexpr int NMF = C::MT * C::NT;
    constexpr int NRD = C::MT + 2 * C::NT;
    constexpr int H = NMF / 2;
    constexpr int R = H / NRD > 0 ? H / NRD : 1;
    constexpr bool BARRIER = ks + 1 == C::KS && (!FINAL || S + 1 < C::STAGES);
    if constexpr (C::SCHED == 1) {
        // position of this k-step's first MFMA in window S-1
        constexpr int OFF = H + ks * NMF;
        if constexpr (!BARRIER) {
            if constexpr (ks + 1 < C::KS)
                read_frags<C>(a_stage<C, S>(smem), b_stage<C, S>(smem), ks + 1, st.a_off,
                              st.b_off, st.fa[1 - P], st.fb[1 - P]);
            mfma_window<C, S - 1, OFF, 0, NMF>(p, ld, kt0, nk, n0, st.fa[P], st.fb[P], st.acc);
        } else {
            constexpr int SN = (S + 1) % C::STAGES;
            mfma_window<C, S - 1, OFF, 0, H>(p, ld, kt0, nk, n0, st.fa[P], st.fb[P], st.acc);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<(C::STAGES - 2) * C::LOADS>();   // my copies of the next step landed
            lds_barrier();                               // everyone's did; stage S is free
            read_frags<C>(a_stage<C, SN>(smem), b_stage<C, SN>(smem), 0, st.a_off, st.b_off,
                          st.fa[1 - P], st.fb[1 - P]);
            mfma_window<C, S, 0, H, NMF>(p, ld, kt0, nk, n0, st.fa[P], st.fb[P], st.acc);
        }
    } else if constexpr (ks + 1 < C::KS) {
        // next k-step of the same K step: prefetch its fragments
        read_frags<C>(a_stage<C, S>(smem), b_stage<C, S>(smem), ks + 1, st.a_off, st.b_off,
                      st.fa[1 - P], st.fb[1 - P]);
        mfma_range<C, 0, NMF>(st.fa[P], st.fb[P], st.acc);
        sched_interleave_reads<NRD, R>();
    } else if constexpr (BARRIER) {
        constexpr int SN = (S + 1) % C::STAGES;
        mfma_range<C, 0, H>(st.fa[P], st.fb[P], st.acc);
        wait_vmcnt<(C::STAGES - 2) * C::LOADS>();   // my copies of the next step landed
        lds_barrier();                               // everyone's did; stage S is free
        read_frags<C>(a_stage<C, SN>(smem), b_stage<C, SN>(smem), 0, st.a_off, st.b_off,
                      st.fa[1 - P], st.fb[1 - P]);
        ld.template issue<S>(p, kt0 + S + C::STAGES, nk, n0);
        mfma_range<C, H, NMF>(st.fa[P], st.fb[P], st.acc);
        sched_interleave_reads<NRD, R>();
    } else {
        mfma_range<C, 0, NMF>(st.fa[P], st.fb[P], st.acc);
    }
}

// Copies the prologue issues after those of K step 0.
template <class C>
constexpr int prologue_after_step0()
{
    if constexpr (C::SCHED == 1) {
        int early = 0;
        for (int t = 0; t < C::LOADS; t++)
            early += Spread<C>::pos(t) < Spread<C>::H;
        return (C::STAGES - 2) * C::LOADS + early;
    } else {
        return (C::STAGES - 1) * C::LOADS;
    }
}

template <class C, bool FINAL, int U = 0>
__device__ __forceinline__ void pipe_body(const Params &p, DirectLoader<C> &ld, const char *smem,
                                          int kt0, int nk, int n0, PipeState<C> &st)
{
    if constexpr (U < C::STAGES * C::KS) {
        pipe_kstep<C, U, FINAL>(p, ld, smem, kt0, nk, n0, st);
        pipe_body<C, FINAL, U + 1>(p, ld, smem, kt0, nk, n0, st);
    }
}

template <class C, typename OutT, bool BIAS>
__global__ void __launch_bounds__(C::THREADS, 1) gemm_pipe(Params p)
{
    static_assert((C::STAGES * C::KS) % 2 == 0, "register double buffer parity per loop body");
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
    int tm, tn;
    tile_coords(p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    PipeState<C> st;
#pragma unroll
    for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int j = 0; j < C::NT; j++)
            st.acc[i][j] = typename C::acc_t{};

    const int nk = (p.K + C::BK - 1) / C::BK;
    if (nk > 0) {
        fragment_offsets<C>(wm, wn, st.a_off, st.b_off);
        DirectLoader<C> ld;
        ld.init(p, smem, m0, n0);
        if constexpr (C::SCHED == 1) {
            // steps 0 .. STAGES-2 whole; of step STAGES-1 the copies whose
            // window position precedes the loop (the rest come from window -1
            // of the first loop body)
            [&]<int... S>(std::integer_sequence<int, S...>) {
                (ld.template issue<S>(p, S, nk, n0), ...);
            }(std::make_integer_sequence<int, C::STAGES - 1>{});
            [&]<int... T>(std::integer_sequence<int, T...>) {
                ((Spread<C>::pos(T) < Spread<C>::H
                      ? ld.template issue_one<C::STAGES - 1, T>(p, C::STAGES - 1, nk, n0)
                      : void()),
                 ...);
            }(std::make_integer_sequence<int, C::LOADS>{});
        } else {
            [&]<int... S>(std::integer_sequence<int, S...>) {
                (ld.template issue<S>(p, S, nk, n0), ...);
            }(std::make_integer_sequence<int, C::STAGES>{});
        }
        wait_vmcnt<prologue_after_step0<C>()>();   // step 0 landed
        lds_barrier();
        read_frags<C>(a_stage<C, 0>(smem), b_stage<C, 0>(smem), 0, st.a_off, st.b_off, st.fa[0],
                      st.fb[0]);
        const int nsteps = (nk + C::STAGES - 1) / C::STAGES * C::STAGES;
        int kt = 0;
        for (; kt + C::STAGES < nsteps; kt += C::STAGES)
            pipe_body<C, false>(p, ld, smem, kt, nk, n0, st);
        pipe_body<C, true>(p, ld, smem, kt, nk, n0, st);
        // drain the dummy copies (they write zeros into LDS) and let every
        // wave finish its fragment reads before LDS is reused for the epilogue
        wait_vmcnt<0>();
        lds_barrier();
    }
    epilogue<C, OutT, BIAS>(p, smem, m0 + wm * C::TM, n0 + wn * C::TN, st.acc);
}

// ============================================================================
// General path: register-staged copies; any pointer alignment (2-byte) and any
// leading dimensions.  Whole 16-byte chunks are read with one unaligned vector
// load (the memory system serves misaligned vector loads of global memory);
// chunks that cross the K or N edge are read element by element.  Same LDS
// layout and fragment reads as the direct path, two LDS stages.
// ============================================================================
template <class C>
struct StagedLoader {
    half8 r[C::LOADS];     // one K step of this thread's chunks: A first, then B
    uint32_t off[C::LOADS];  // element offset of each chunk from the tile corner
                           // (host: bm * lda and bk * ldb stay below 2^31)

    __device__ __forceinline__ static int a_row(int t)
    {
        return ((threadIdx.x >> 6) * C::A_LOADS + t) * C::A_ROWS_PER_LOAD +
               (threadIdx.x & 63) / (C::BK / 8);
    }
    __device__ __forceinline__ static int a_kc(int t)
    {
        return (((threadIdx.x & 63) % (C::BK / 8)) ^ swz_a<C::BK>(a_row(t))) * 8;
    }
    __device__ __forceinline__ static int b_k(int t)
    {
        return ((threadIdx.x >> 6) * C::B_LOADS + t) * C::B_ROWS_PER_LOAD +
               (threadIdx.x & 63) / (C::BN / 8);
    }
    __device__ __forceinline__ static int b_col(int t)
    {
        return (((threadIdx.x & 63) % (C::BN / 8)) ^ swz_b<C::BN>(b_k(t))) * 8;
    }

    __device__ __forceinline__ void init(const Params &p)
    {
#pragma unroll
        for (int t = 0; t < C::A_LOADS; t++)
            off[t] = (uint32_t)(a_row(t) * p.lda + a_kc(t));
#pragma unroll
        for (int t = 0; t < C::B_LOADS; t++)
            off[C::A_LOADS + t] = (uint32_t)(b_k(t) * p.ldb + b_col(t));
    }

    // Load K step kt into registers; zeros past M, N and K (so steps past the
    // end load zeros).  Whole 16-byte chunks are one unaligned vector load.
    __device__ __forceinline__ void load(const Params &p, int m0, int n0, int kt)
    {
        const int k0 = kt * C::BK;
        const _Float16 *a0 = p.A + (int64_t)m0 * p.lda + k0;
        const _Float16 *b0 = p.B + (int64_t)k0 * p.ldb + n0;
        if (m0 + C::BM <= p.M && n0 + C::BN <= p.N && k0 + C::BK <= p.K) {
            // interior: every chunk is whole
#pragma unroll
            for (int t = 0; t < C::LOADS; t++)
                __builtin_memcpy(&r[t], (t < C::A_LOADS ? a0 : b0) + off[t], 16);
            return;
        }
#pragma unroll
        for (int t = 0; t < C::A_LOADS; t++) {
            const int kleft = p.K - k0 - a_kc(t);   // valid elements of the chunk
            half8 v = {};
            if (m0 + a_row(t) < p.M && kleft > 0) {
                const _Float16 *src = a0 + off[t];
                if (kleft >= 8) {
                    __builtin_memcpy(&v, src, 16);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        v[e] = e < kleft ? src[e] : (_Float16)0.f;
                }
            }
            r[t] = v;
        }
#pragma unroll
        for (int t = 0; t < C::B_LOADS; t++) {
            const int nleft = p.N - n0 - b_col(t);
            half8 v = {};
            if (k0 + b_k(t) < p.K && nleft > 0) {
                const _Float16 *src = b0 + off[C::A_LOADS + t];
                if (nleft >= 8) {
                    __builtin_memcpy(&v, src, 16);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        v[e] = e < nleft ? src[e] : (_Float16)0.f;
                }
            }
            r[C::A_LOADS + t] = v;
        }
    }

    // Registers -> LDS stage S, in the layout the direct copies produce.
    template <int S>
    __device__ __forceinline__ void store(char *smem) const
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int t = 0; t < C::A_LOADS; t++)
            *(half8 *)(smem + S * C::A_BYTES + (wave * C::A_LOADS + t) * 1024 + lane * 16) = r[t];
#pragma unroll
        for (int t = 0; t < C::B_LOADS; t++)
            *(half8 *)(smem + C::STAGES * C::A_BYTES + S * C::B_BYTES +
                       (wave * C::B_LOADS + t) * 1024 + lane * 16) = r[C::A_LOADS + t];
    }
};

// k-step U of a loop body of the register-staged kernel (two LDS stages).
// The loads of K step j+1 are issued right after the barrier that starts K
// step j and written to LDS in the first half of the last k-step of step j,
// before the barrier that publishes them.  LAST: the k-step that ends the K
// loop.
template <class C, int U, bool LAST>
__device__ __forceinline__ void staged_kstep(const Params &p, StagedLoader<C> &ld, char *smem,
                                             int kt0, int nk, int m0, int n0, PipeState<C> &st)
{
    constexpr int S = U / C::KS, ks = U % C::KS, P = U % 2;
    constexpr int NMF = C::MT * C::NT;
    constexpr int NRD = C::MT + 2 * C::NT;
    constexpr int H = NMF / 2;
    constexpr int R = H / NRD > 0 ? H / NRD : 1;
    if constexpr (ks + 1 < C::KS) {
        read_frags<C>(a_stage<C, S>(smem), b_stage<C, S>(smem), ks + 1, st.a_off, st.b_off,
                      st.fa[1 - P], st.fb[1 - P]);
        mfma_range<C, 0, NMF>(st.fa[P], st.fb[P], st.acc);
        sched_interleave_reads<NRD, R>();
    } else if constexpr (!LAST) {
        constexpr int SN = (S + 1) % 2;
        mfma_range<C, 0, H>(st.fa[P], st.fb[P], st.acc);
        ld.template store<SN>(smem);                 // K step kt0+S+1 (its stage is free)
        lds_barrier();                               // publishes it; stage S is free
        read_frags<C>(a_stage<C, SN>(smem), b_stage<C, SN>(smem), 0, st.a_off, st.b_off,
                      st.fa[1 - P], st.fb[1 - P]);
        if (kt0 + S + 2 < nk)
            ld.load(p, m0, n0, kt0 + S + 2);
        mfma_range<C, H, NMF>(st.fa[P], st.fb[P], st.acc);
        sched_interleave_reads<NRD, R>();
    } else {
        mfma_range<C, 0, NMF>(st.fa[P], st.fb[P], st.acc);
    }
}

// NS K steps (1 or 2) from kt0; LASTBODY: the K loop ends with this body.
template <class C, int NS, bool LASTBODY, int U = 0>
__device__ __forceinline__ void staged_body(const Params &p, StagedLoader<C> &ld, char *smem,
                                            int kt0, int nk, int m0, int n0, PipeState<C> &st)
{
    if constexpr (U < NS * C::KS) {
        staged_kstep<C, U, LASTBODY && U + 1 == NS * C::KS>(p, ld, smem, kt0, nk, m0, n0, st);
        staged_body<C, NS, LASTBODY, U + 1>(p, ld, smem, kt0, nk, m0, n0, st);
    }
}

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

    PipeState<C> st;
#pragma unroll
    for (int i = 0; i < C::MT; i++)
#pragma unroll
        for (int j = 0; j < C::NT; j++)
            st.acc[i][j] = typename C::acc_t{};

    const int nk = (p.K + C::BK - 1) / C::BK;
    if (nk > 0) {
        fragment_offsets<C>(wm, wn, st.a_off, st.b_off);
        StagedLoader<C> ld;
        ld.init(p);
        ld.load(p, m0, n0, 0);
        ld.template store<0>(smem);
        if (nk > 1)
            ld.load(p, m0, n0, 1);
        lds_barrier();
        read_frags<C>(a_stage<C, 0>(smem), b_stage<C, 0>(smem), 0, st.a_off, st.b_off, st.fa[0],
                      st.fb[0]);
        // bodies of two K steps; an odd count ends with a one-step body (the
        // register parity of a body is even when KS is even, and a one-step
        // body is only ever the last)
        int kt = 0;
        for (; kt + 2 < nk; kt += 2)
            staged_body<C, 2, false>(p, ld, smem, kt, nk, m0, n0, st);
        if (nk - kt == 2)
            staged_body<C, 2, true>(p, ld, smem, kt, nk, m0, n0, st);
        else
            staged_body<C, 1, true>(p, ld, smem, kt, nk, m0, n0, st);
        lds_barrier();   // every wave past its last fragment read
    }
    epilogue<C, OutT, BIAS>(p, smem, m0 + wm * C::TM, n0 + wn * C::TN, st.acc);
}

// ------------------------------------------------------------ instances --
template <class C, int KIND>
hipError_t launch_cfg(const Params &p, bool f16_out, bool bias, hipStream_t s)
{
    const dim3 grid(p.tiles_m * p.tiles_n), block(C::THREADS);
#define TG_GO(KERNEL, OUT, B)                                                        \
    do {                                                                             \
        hipLaunchKernelGGL((KERNEL<C, OUT, B>), grid, block, 0, s, p);               \
        return hipGetLastError();                                                    \
    } while (0)
    if constexpr (KIND == 2) {
        if (f16_out) { if (bias) TG_GO(gemm_pipe, _Float16, true); else TG_GO(gemm_pipe, _Float16, false); }
        else { if (bias) TG_GO(gemm_pipe, float, true); else TG_GO(gemm_pipe, float, false); }
    } else {
        if (f16_out) { if (bias) TG_GO(gemm_staged, _Float16, true); else TG_GO(gemm_staged, _Float16, false); }
        else { if (bias) TG_GO(gemm_staged, float, true); else TG_GO(gemm_staged, float, false); }
    }
#undef TG_GO
}

// The library is built from TG_SHARDS compilations of this file (so they
// can run in parallel); compilation TG_SHARD instantiates the configurations
// whose id is TG_SHARD modulo TG_SHARDS and publishes their launchers in its
// own table.  Compilation 0 also holds the description table.
#ifndef TG_SHARD
#define TG_SHARD 0
#endif
#ifndef TG_SHARDS
#define TG_SHARDS 1
#endif
static_assert(TG_SHARDS >= 1 && TG_SHARDS <= kMaxShards && TG_SHARD < TG_SHARDS, "shards");

template <int ID, class CFG, int KIND>
LaunchFn shard_launch()
{
    if constexpr (ID % TG_SHARDS == TG_SHARD)
        return &launch_cfg<CFG, KIND>;
    else
        return nullptr;
}

#define TG_CAT2(a, b) a##b
#define TG_CAT(a, b) TG_CAT2(a, b)

// The launch tables are host data (the device pass would otherwise turn the
// const arrays into device constant memory).
#if !defined(__HIP_DEVICE_COMPILE__)
// every shard's table, weakly referenced: shards beyond TG_SHARDS do not exist
#define TG_SHARD_DECL(i) extern const LaunchFn kShardLaunch##i[] __attribute__((weak));
TG_SHARD_DECL(0) TG_SHARD_DECL(1) TG_SHARD_DECL(2) TG_SHARD_DECL(3)
TG_SHARD_DECL(4) TG_SHARD_DECL(5) TG_SHARD_DECL(6) TG_SHARD_DECL(7)
#undef TG_SHARD_DECL

#define TG_CONFIG_ROW(ID, BM, BN, BK, WM, WN, ST, MI, KIND, SCH)                          \
    shard_launch<ID, Cfg<BM, BN, BK, WM, WN, ST, MI, SCH>, KIND>(),
const LaunchFn TG_CAT(kShardLaunch, TG_SHARD)[] = {
#include "tg_config_list.inc"
};
#undef TG_CONFIG_ROW
#else
// device pass: instantiate the kernels of this shard
#define TG_CONFIG_ROW(ID, BM, BN, BK, WM, WN, ST, MI, KIND, SCH)                          \
    template LaunchFn shard_launch<ID, Cfg<BM, BN, BK, WM, WN, ST, MI, SCH>, KIND>();
#include "tg_config_list.inc"
#undef TG_CONFIG_ROW
#endif

#if TG_SHARD == 0 && !defined(__HIP_DEVICE_COMPILE__)
#define TG_CONFIG_ROW(ID, BM, BN, BK, WM, WN, ST, MI, KIND, SCH)                          \
    {ID, BM, BN, BK, ST, WM, WN, MI, (KIND) != 0,                                    \
     Cfg<BM, BN, BK, WM, WN, ST, MI, SCH>::LDS_BYTES,                                     \
     (KIND == 2 ? "pipe_" #BM "x" #BN "x" #BK "_s" #ST "_w" #WM "x" #WN "_mi" #MI    \
                      "_c" #SCH                                                      \
                : "staged_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_mi" #MI)},

const KernelConfig kConfigs[] = {
#include "tg_config_list.inc"
};
const int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
#undef TG_CONFIG_ROW

LaunchFn config_launch(int id)
{
    static const LaunchFn *const shards[kMaxShards] = {
        kShardLaunch0, kShardLaunch1, kShardLaunch2, kShardLaunch3,
        kShardLaunch4, kShardLaunch5, kShardLaunch6, kShardLaunch7};
    if (id < 0 || id >= kNumConfigs)
        return nullptr;
    for (int s = 0; s < kMaxShards; s++)
        if (shards[s] && shards[s][id])
            return shards[s][id];
    return nullptr;
}
#endif

}  // namespace tg
