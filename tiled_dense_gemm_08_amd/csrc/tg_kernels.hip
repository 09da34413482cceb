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

#include <type_traits>
#include <utility>

#include "tg_kernels.h"

namespace tg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));

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

// s_waitcnt lgkmcnt(0): this wave's LDS writes have completed.
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

#ifdef TG_LDS_POISON
// Debug builds (-DTG_LDS_POISON): LDS is filled with fp16 NaN (all ones)
// before it is written, so that an LDS read of bytes that no copy of the
// current K step wrote -- a stage read before its copies landed, or a copy
// that leaves bytes untouched -- reaches the MFMAs as NaN and shows in C.
__device__ __forceinline__ void poison16(uint32_t lds)
{
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    *(__attribute__((address_space(3))) u4 *)(uintptr_t)lds = u4{~0u, ~0u, ~0u, ~0u};
}

// The whole of a workgroup's LDS, at kernel start.
template <int BYTES, int THREADS>
__device__ __forceinline__ void poison_all(char *smem)
{
    const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
    for (int i = threadIdx.x; i < BYTES / 16; i += THREADS)
        poison16(base + 16 * i);
    __syncthreads();
}
#endif

// ---------------------------------------------------------------- swizzles --
// A tile in LDS: BM rows of BK fp16 (k contiguous), 16-byte chunks XOR-
// swizzled by row.  A fragment read has MI lanes on MI consecutive rows at
// the same logical chunk.  With 128-byte rows, XOR by (row & 7) reads at the
// full ds_read_b128 rate on gfx950 (measured: about 200 B/clk/CU, against
// about 60 without a swizzle).  64-byte rows (BK = 32) use a 2-bit analogue.
// Both are unchanged by row += 16, so one per-lane offset serves every block.
template <int ROWB>
__device__ __forceinline__ int swz_a(int row)
{
    static_assert(ROWB == 128 || ROWB == 64, "k-major row bytes");
    if constexpr (ROWB == 128)
        return row & 7;
    else
        return (row >> 1) & 3;
}

// B tile in LDS: BK rows of BN fp16 (n contiguous).  A transpose read has, per
// 16-lane group, 4 rows (k % 4 = 0..3) of 32 bytes, and groups sit on rows 8
// apart; the swizzle (multiples of 2 chunks, so the 32-byte pairs stay whole)
// spreads rows {0..3, 8..11} over 8 distinct 32-byte slots.  It must stay
// below the BN/8 chunks of a row: a 64-wide row is 128 bytes, half of the
// banks, so rows of either parity share the 4 slots of their half, and the
// swizzle on k bits 1 and 3 gives each slot 2 of the 16 rows a read touches
// (XOR by k % 4 alone gave 4: the groups 8 rows apart coincided).  Both are
// unchanged by k += 4, 16 and 32.
template <int BN>
__device__ __forceinline__ int swz_b(int k)
{
    if constexpr (BN >= 128)
        return 2 * (k & 3) + 8 * ((k >> 3) & 1);
    else
        return 2 * ((k >> 1) & 1) + 4 * ((k >> 3) & 1);
}

// Same for 1-byte elements (R bytes per row): the 8-bit transpose read has,
// per 16-lane group, 8 rows (k % 8 = 0..7) of 16 bytes; XOR by k % 8 puts them
// on 8 distinct 16-byte slots.  The groups sit 16 rows apart: with 256-byte
// rows (16 slots) k bit 4 also moves to the other half of the row, so that
// neighbouring groups do not land on the same banks (bank conflicts per
// active LDS cycle on 8192^3 int8: 0.25 with k % 8 alone).  Unchanged by
// k += 8 and k += 64.
template <int R>
__device__ __forceinline__ int swz_b8(int k)
{
    constexpr int CHUNKS = R / 16;
    if constexpr (CHUNKS >= 16)
        return (k & 7) ^ (8 * ((k >> 4) & 1));
    else
        return k & (CHUNKS >= 8 ? 7 : CHUNKS - 1);
}

// The swizzle of an mn-major tile of R elements of ES bytes per row.
template <int ES, int R>
__device__ __forceinline__ int swz_mn(int k)
{
    if constexpr (ES == 2)
        return swz_b<R>(k);
    else
        return swz_b8<R>(k);
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
template <int MI, int ES> struct AccT;
template <> struct AccT<16, 2> { typedef float4v type; };
template <> struct AccT<32, 2> { typedef float16v type; };
template <> struct AccT<16, 1> { typedef int4v type; };
template <> struct AccT<32, 1> { typedef int16v type; };

// ES: operand element size: 2 (fp16 operands, fp32 accumulation) or 1 (int8
// operands, int32 accumulation).  BK counts elements; a k-major tile row is
// BK * ES bytes (64 or 128), and every copy, swizzle and fragment read works
// on 16-byte chunks, so both element sizes share them.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int STAGES_, int MI_, int SCHED_,
          int TA_ = 0, int TB_ = 0, int ES_ = 2>
struct Cfg {
    static constexpr int ES = ES_;
    // copy issue: 0 burst after the barrier, 1 spread, 2 interleaved with the
    // MFMA rows that follow the barrier, 3 spread as in 1 with the next
    // k-step's fragment reads placed one by one between the MFMAs and the
    // MFMAs written as assembly on accumulators pinned to their registers
    // (the one-wave-per-SIMD 16x16x32 kernels, see mfma()).  With A stored
    // K x M (TA) schedule 2 spills registers inside the K loop (an mn-major A
    // block is two transpose reads and has its own offset register), so
    // those orientations keep schedule 0.
    static constexpr int SCHED = SCHED_ == 2 && TA_ ? 0 : SCHED_;
    // Operand orientation: TA = 1 when A is stored K x M (the product uses its
    // transpose), TB = 1 when B is stored N x K.  The LDS tile of an operand is
    // k-major (rows of BK fp16, k contiguous, read with ds_read_b128) when its
    // rows run along M or N in memory, and mn-major (BK rows, M or N
    // contiguous, read with the transpose read) otherwise.
    static constexpr bool TA = TA_ != 0, TB = TB_ != 0;
    static constexpr bool A_KMAJ = !TA, B_KMAJ = TB;
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WM_, WAVES_N = WN_;
    static constexpr int STAGES = STAGES_;
    static constexpr int MI = MI_;                         // MFMA block edge
    static constexpr int KI = 1024 / MI / ES;              // k per MFMA: 32x32: 16 (fp16), 32 (int8)
    static constexpr int ACC = MI * MI / 64;               // accumulators per lane per block
    static constexpr int WAVES = WM_ * WN_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TM = BM / WM_, TN = BN / WN_;     // wave tile
    static constexpr int MT = TM / MI, NT = TN / MI;       // MFMA blocks per wave
    static constexpr int KS = BK / KI;                     // MFMA k-steps per K step
    // A fragments single-buffered and refilled row by row (pipe_kstep_roll):
    // the 16x16x32 MFMA needs twice the fragment registers of 32x32x16 for
    // the same wave tile, and with two waves per SIMD (8 waves) the double-
    // buffered set would not fit in a wave's 256 registers.  SCHED 2 is the
    // rolling kernel with the work that follows each barrier (next
    // fragments, refill copies) interleaved with the MFMAs that need no new
    // data instead of issued ahead of them (post_barrier_rows).
    static constexpr bool ROLL = MI_ == 16 && WM_ * WN_ == 8 && (SCHED_ == 0 || SCHED_ == 2);
    // Schedule 3 serves only K that is a whole number of K steps (the host
    // checks it): its copies then need no per-lane test for chunks past K,
    // an instruction per copy that its single wave per SIMD would pay for.
    static constexpr bool WHOLE_K = SCHED_ == 3;
    static constexpr int A_BYTES = BM * BK * ES;
    static constexpr int B_BYTES = BK * BN * ES;
    static constexpr int KROWB = BK * ES;                  // bytes of a k-major tile row
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    // global->LDS copy: each wave instruction moves 1 KiB (64 lanes x 16 B)
    static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;  // per thread per K step
    static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    // rows of the LDS tile that one copy instruction (1 KiB) fills
    static constexpr int A_ROWS_PER_LOAD = A_KMAJ ? 1024 / KROWB : 1024 / (BM * ES);
    static constexpr int B_ROWS_PER_LOAD = B_KMAJ ? 1024 / KROWB : 1024 / (BN * ES);
    // fragment offset registers: one per k-step (k-major) or per block (mn-major)
    static constexpr int A_NOFF = A_KMAJ ? BK / KI : BM / WM_ / MI_;
    static constexpr int B_NOFF = B_KMAJ ? BK / KI : BN / WN_ / MI_;
    typedef typename AccT<MI, ES>::type acc_t;
    static_assert(MI == 16 || MI == 32, "MI");
    static_assert(ES == 1 || ES == 2, "element size");
    static_assert(KROWB == 64 || KROWB == 128, "BK");
    static_assert(TM % MI == 0 && TN % MI == 0, "wave tile");
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0, "copy split");
    static_assert(BN * ES <= 1024 && BN % 64 == 0 && BM * ES <= 1024 && BM % 64 == 0, "BM, BN");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// ------------------------------------------------------------- fragments --
// Per-lane LDS byte offsets of the fragment reads (stage-relative).  An MFMA
// operand fragment gives lane l the 8 k = 8 (l / MI) .. +7 of the k-step for
// row (A, second source) or column (B, first source) l % MI of its block.
//  k-major tile (R rows of BK): one ds_read_b128 per block at
//    off[ks] + block * MI * BK * ES.
//  mn-major tile (BK rows of R), fp16: two transpose reads of 4 k each: lane
//    L = 16 G + 4 e + q reads row k = 8 (L / MI) + e (+4 for the second read,
//    + KI per k-step) at positions 16 ((L % MI) / 16) + 4 q .. +3 of the
//    block; the hardware hands lane 16 G + j the 4 rows' position j.
//  mn-major tile, int8: two 8-bit transpose reads of 8 k each: lane
//    L = 16 G + 2 e + h reads row k = 16 (L / MI) + e (+8 for the second read)
//    at positions 16 ((L % MI) / 16) + 8 h .. +7; lane 16 G + j receives the 8
//    rows' position j (measured on gfx950 with an in-bounds probe).
//    off[block] + ks * KI * R * ES.
template <class C, int NOFF>
__device__ __forceinline__ void kmajor_offsets(int base, int (&off)[NOFF])
{
    const int lane = threadIdx.x & 63;
    const int row = base + lane % C::MI;
#pragma unroll
    for (int ks = 0; ks < NOFF; ks++) {
        const int chunk = ks * (C::KI * C::ES / 16) + lane / C::MI;
        off[ks] = row * C::KROWB + ((chunk ^ swz_a<C::KROWB>(row)) * 16);
    }
}

template <class C, int R, int NOFF>
__device__ __forceinline__ void mnmajor_offsets(int base, int (&off)[NOFF])
{
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const int sub = (lane % C::MI) >> 4;
    if constexpr (C::ES == 2) {
        const int e = i >> 2, q = i & 3;
        const int k = 8 * (lane / C::MI) + e;
#pragma unroll
        for (int b = 0; b < NOFF; b++) {
            const int col = base + b * C::MI + sub * 16 + 4 * q;
            off[b] = k * R * 2 + (((col >> 3) ^ swz_b<R>(k)) * 16) + (col & 7) * 2;
        }
    } else {
        const int e = i >> 1, h = i & 1;
        const int k = 16 * (lane / C::MI) + e;
#pragma unroll
        for (int b = 0; b < NOFF; b++) {
            const int col = base + b * C::MI + sub * 16 + 8 * h;
            off[b] = k * R + (((col >> 4) ^ swz_b8<R>(k)) * 16) + (col & 15);
        }
    }
}

template <class C>
__device__ __forceinline__ void fragment_offsets(int wm, int wn, int (&a_off)[C::A_NOFF],
                                                 int (&b_off)[C::B_NOFF])
{
    if constexpr (C::A_KMAJ)
        kmajor_offsets<C>(wm * C::TM, a_off);
    else
        mnmajor_offsets<C, C::BM>(wm * C::TM, a_off);
    if constexpr (C::B_KMAJ)
        kmajor_offsets<C>(wn * C::TN, b_off);
    else
        mnmajor_offsets<C, C::BN>(wn * C::TN, b_off);
}

template <class C, bool KMAJ, int R, int NOFF>
__device__ __forceinline__ half8 read_block(const char *tile, int ks, const int (&off)[NOFF], int b)
{
    if constexpr (KMAJ) {
        return *(const half8 *)(tile + off[ks] + b * C::MI * C::KROWB);
    } else if constexpr (C::ES == 2) {
        const char *q = tile + off[b] + ks * C::KI * R * 2;
        short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v *)TG_LDS(q));
        short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v *)TG_LDS(q + 4 * R * 2));
        return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
        const char *q = tile + off[b] + ks * C::KI * R;
        int2v lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) int2v *)TG_LDS(q));
        int2v hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) int2v *)TG_LDS(q + 8 * R));
        return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3));
    }
}

template <class C, bool KMAJ, int R, int NOFF, int NBLK>
__device__ __forceinline__ void read_operand(const char *tile, int ks, const int (&off)[NOFF],
                                             half8 (&frag)[NBLK])
{
#pragma unroll
    for (int b = 0; b < NBLK; b++)
        frag[b] = read_block<C, KMAJ, R>(tile, ks, off, b);
}

// B fragments first (transpose reads in the normal orientation), then A.
template <class C>
__device__ __forceinline__ void read_frags(const char *as, const char *bs, int ks,
                                           const int (&a_off)[C::A_NOFF],
                                           const int (&b_off)[C::B_NOFF], half8 (&fa)[C::MT],
                                           half8 (&fb)[C::NT])
{
    read_operand<C, C::B_KMAJ, C::BN>(bs, ks, b_off, fb);
    read_operand<C, C::A_KMAJ, C::BM>(as, ks, a_off, fa);
}

// half8 is the 16-byte fragment container for both element sizes.
//
// Schedule 3 issues the 16x16x32 MFMA as assembly with the accumulator tied
// in place ("+a": the same accumulation registers in and out).  A wave of
// these kernels holds a 128 x 128 fp32 tile, all 256 accumulation registers;
// with the builtin and the fragment reads placed between the MFMAs, the
// register allocator moved hundreds of accumulator registers per loop body
// through the other registers.  The compiler does not see these MFMAs, so the
// kernel keeps their hazards itself: the fragment registers they read come
// from LDS reads that the compiler's waits cover, each accumulator is
// written by one MFMA per k-step (64 MFMAs apart), and acc_fence() puts wait
// states between the accumulators' other writers and readers and the MFMAs.
template <class C>
__device__ __forceinline__ typename C::acc_t mfma(half8 b, half8 a, typename C::acc_t c)
{
    if constexpr (C::ES == 2 && C::MI == 16 && C::SCHED == 3) {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
        return c;
    } else if constexpr (C::ES == 1 && C::MI == 16 && C::SCHED == 3) {
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
        return c;
    } else if constexpr (C::ES == 1) {
        const int4v bi = __builtin_bit_cast(int4v, b), ai = __builtin_bit_cast(int4v, a);
        if constexpr (C::MI == 16)
            return __builtin_amdgcn_mfma_i32_16x16x64_i8(bi, ai, c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_i32_32x32x32_i8(bi, ai, c, 0, 0, 0);
    } else if constexpr (C::MI == 16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0);
    }
}

// Schedule 3: wait states between the assembly MFMAs and the compiler's own
// accesses of the accumulators (their zeroing before the K loop, their reads
// in the epilogue).  Every accumulator passes through an empty statement
// ordered after (AFTER) or before the s_nop, so no such access can move to
// the other side of it; 48 wait states cover the longest MFMA-to-VALU rule
// of the 16x16x32 shape.
template <class C, bool AFTER>
__device__ __forceinline__ void acc_fence(typename C::acc_t (&acc)[C::MT][C::NT])
{
    if constexpr (C::SCHED == 3) {
        if constexpr (AFTER)
            asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15");
#pragma unroll
        for (int i = 0; i < C::MT; i++)
#pragma unroll
            for (int j = 0; j < C::NT; j++)
                asm volatile("" : "+a"(acc[i][j]));
        if constexpr (!AFTER)
            asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15");
    }
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

// 4 accumulator values of one run: fp32 (fp16 operands) or int32 (int8).
template <class C>
using val4_t = typename std::conditional<C::ES == 1, int4v, float4v>::type;

template <class C, bool BIAS>
__device__ __forceinline__ val4_t<C> epi_value(const typename C::acc_t &a, int run, float4v bv)
{
    val4_t<C> v;
#pragma unroll
    for (int r = 0; r < 4; r++)
        v[r] = a[4 * run + r];
    if constexpr (BIAS) {
        static_assert(C::ES == 2, "bias + ReLU is an fp32 epilogue");
#pragma unroll
        for (int r = 0; r < 4; r++)
            v[r] = fmaxf(v[r] + bv[r], 0.f);
    }
    return v;
}

// Store 4 consecutive outputs: fp32 and int32 as 16 bytes, fp16 converted
// (round to nearest even) as 8 bytes.
template <typename OutT, typename V>
__device__ __forceinline__ void store4(char *dst, V v)
{
    if constexpr (sizeof(OutT) == 4) {
        *(V *)dst = v;
    } else {
        half4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        *(half4 *)dst = h;
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

// Epilogue: the wave writes its converted tile, PR rows at a time, into a
// private LDS region in row-major order (rows padded by 16 bytes so that the
// 32 rows one MFMA block spans spread over the banks), then reads it back so
// that consecutive lanes hold consecutive 16-byte chunks of a row, and stores
// those: every store instruction writes runs of whole 128-byte lines of C
// instead of 16 bytes in each of 32 rows.  A row of C that does not start on
// a 16-byte boundary (leading dimension or base not a multiple of 16 bytes)
// takes the same 16-byte stores, misaligned (the memory system serves
// misaligned vector stores to global memory); its runs then straddle one
// more line.  The row's last, partial chunk is stored element by element.
// The caller has made the workgroup's LDS free (no copy in flight, every
// wave past its last fragment read).
template <class C, typename OutT, bool BIAS>
__device__ __forceinline__ void epilogue(const Params &p, char *smem, int m_base, int n_base,
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
    constexpr int NIT = PR * CPR / 64;                     // read-back instructions per pass
    constexpr int BATCH = NIT < 4 ? NIT : 4;
    static_assert(NIT % BATCH == 0, "whole read-back batches");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    char *region = smem + wave * REGION;
    // every row of C starts on a 16-byte boundary (so do the wave tile's
    // 16-byte chunks: its first column is a multiple of 8 elements)
    const bool c_lines = ((uintptr_t)p.C & 15) == 0 && (p.ldc * ES) % 16 == 0;

    // The bias of the lane's columns, loaded once for every pass: with the
    // wave tile's columns inside N and a 16-byte aligned bias
    // (wave-uniform), as 16-byte loads that one wait covers.
    float4v bvs[BIAS ? C::NT : 1][BIAS ? RUNS : 1];
    if constexpr (BIAS) {
        if (p.vec_bias && n_base + C::TN <= p.N) {
#pragma unroll
            for (int nt = 0; nt < C::NT; nt++)
#pragma unroll
                for (int run = 0; run < RUNS; run++)
                    bvs[nt][run] = *(const float4v *)(p.bias + n_base + run_col<C>(nt, run));
        } else {
#pragma unroll
            for (int nt = 0; nt < C::NT; nt++)
#pragma unroll
                for (int run = 0; run < RUNS; run++)
                    bvs[nt][run] = load_bias4(p, n_base + run_col<C>(nt, run));
        }
    }

#pragma unroll
    for (int pass = 0; pass < C::TM / PR; pass++) {
        // registers -> LDS (row-major, padded rows)
#pragma unroll
        for (int nt = 0; nt < C::NT; nt++)
#pragma unroll
            for (int run = 0; run < RUNS; run++) {
                float4v bv = {0.f, 0.f, 0.f, 0.f};
                if constexpr (BIAS)
                    bv = bvs[nt][run];
#pragma unroll
                for (int i = 0; i < MT_PASS; i++) {
                    const int mt = pass * MT_PASS + i;
                    const int row = i * C::MI + lane % C::MI;
                    const val4_t<C> v = epi_value<C, BIAS>(acc[mt][nt], run, bv);
                    store4<OutT>(region + row * ROWB + run_col<C>(nt, run) * ES, v);
                }
        }
        // LDS -> C, 16 bytes per lane, consecutive lanes along a row.  A wave's
        // LDS accesses complete in order, so no barrier is needed: the region
        // is private to this wave.  The reads go out in batches, outside any
        // bounds test, so that one wait covers a batch.  Where the pass's
        // rows and the wave tile's columns lie wholly inside C and C's rows
        // start on 16-byte boundaries (wave-uniform), the stores take no
        // per-chunk tests and are marked non-temporal: C is not read again
        // here, and a round of tiles writes as much C as an XCD's L2 holds,
        // which as ordinary stores evicts the operand panels the next
        // round's tiles read.  Misaligned rows keep ordinary stores, whose
        // partial lines L2 merges (as non-temporal stores they reached
        // memory separately: 17 % more bytes written).
        const bool stream =
            c_lines && m_base + (pass + 1) * PR <= p.M && n_base + C::TN <= p.N;
#pragma unroll
        for (int b0 = 0; b0 < NIT; b0 += BATCH) {
            float4v v[BATCH];
#pragma unroll
            for (int j = 0; j < BATCH; j++) {
                const int q = (b0 + j) * 64 + lane;
                v[j] = *(const float4v *)(region + (q / CPR) * ROWB + (q % CPR) * 16);
            }
#pragma unroll
            for (int j = 0; j < BATCH; j++) {
                const int q = (b0 + j) * 64 + lane;
                const int r = q / CPR, cc = q % CPR;
                const int row = m_base + pass * PR + r;
                const int col = n_base + cc * (16 / ES);
                OutT *dst = (OutT *)p.C + (int64_t)row * p.ldc + col;
                if (stream) {
                    __builtin_nontemporal_store(v[j], (float4v *)dst);   // 16-byte aligned
                } else if (row < p.M) {
                    if (col + 16 / ES <= p.N) {
                        __builtin_memcpy(dst, &v[j], 16);   // any alignment of the element size
                    } else {
                        const OutT *e = (const OutT *)&v[j];
#pragma unroll
                        for (int i = 0; i < 16 / ES; i++)
                            if (col + i < p.N)
                                dst[i] = e[i];
                    }
                }
            }
        }
    }
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
// kernels; the compiler reserves M0 and is not told of the write (a clobber
// of a reserved register is not honoured), so tests/test_device_asm_cpu.py
// checks the device assembly of every kernel for any other M0 use.  A scalar
// write of M0 needs one wait state before a load that uses it as the LDS
// address.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds)
                 : "memory");
}

// dma16 with the LDS address formed in M0 itself, base + IMM: one scalar
// instruction less per copy (the schedule-3 kernels, one wave per SIMD).
template <uint32_t IMM>
__device__ __forceinline__ void dma16_at(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t base)
{
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(base), "n"(IMM)
                 : "memory", "scc");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)p;
}

// Wave w's copy instruction t of a K step fills LDS bytes [1 KiB * (w *
// LOADS + t), +1 KiB) of an operand's tile: ROWS_PER_LOAD rows of it.  In a
// k-major tile lane i takes row i / (BK/8) and physical chunk i % (BK/8); in an
// mn-major tile k-row i / (R/8) and physical chunk i % (R/8).  The swizzle is
// applied on the global side: each lane fetches the logical chunk that belongs
// at its physical slot.
//
// The K position is carried by the buffer descriptors, not by the lane
// offsets: for K step kt a k-major operand's descriptor starts kt*BK elements
// further along its rows, an mn-major one kt*BK rows further down, with the
// range shortened by as much, so the lane offsets are constants of the tile
// and a K step costs a few scalar instructions.  The range check gives zeros
// for rows past the end of the operand (rows past M or N of a k-major tile,
// rows past K of an mn-major one; the host guarantees those offsets do not
// wrap 32 bits); the columns past K of a k-major tile in the last K step and
// the columns past M or N of an mn-major tile lie inside the buffer and are
// pushed out of range explicitly.  Steps at or past nk get a zero-length
// descriptor: every lane reads zeros without touching memory, so each K step
// keeps the same number of outstanding copies.
template <class C, bool KMAJ, int R, int NLOADS>
struct OperandCopy {
    static constexpr int ES = C::ES;
    static constexpr int RCH = KMAJ ? C::KROWB / 16 : R * ES / 16;   // 16-byte chunks per row
    static constexpr int RPL = 64 / RCH;                             // rows per instruction
    uint32_t lane_off;   // k-major: byte offset of this lane's chunk in instruction 0
    int kc;              // k-major: logical k (elements) of this lane's chunk in the tile
    int row, phys;       // mn-major: k-row within an instruction; physical chunk

    __device__ __forceinline__ void init(int x0, int ld)
    {
        const int lane = threadIdx.x & 63;
        if constexpr (KMAJ) {
            const int r = lane / RCH;
            // the swizzle depends on row % RPL only (8 or 16 rows)
            kc = ((lane % RCH) ^ swz_a<C::KROWB>(r)) * (16 / ES);
            lane_off = (uint32_t)(((int64_t)(x0 + r) * ld + kc) * ES);
        } else {
            row = lane / RCH;
            phys = lane % RCH;
        }
    }

    // Lane byte offset of copy instruction t (x0: tile origin along M or N;
    // X: M or N).
    __device__ __forceinline__ uint32_t off(int t, int x0, int X, int ld) const
    {
        const int inst = (threadIdx.x >> 6) * NLOADS + t;
        if constexpr (KMAJ) {
            return lane_off + (uint32_t)(inst * RPL) * (uint32_t)ld * (uint32_t)ES;
        } else {
            const int k = inst * RPL + row;
            const int col = x0 + (phys ^ swz_mn<ES, R>(k)) * (16 / ES);
            return col < X ? ((uint32_t)k * (uint32_t)ld + (uint32_t)col) * (uint32_t)ES : kOOB;
        }
    }

    // Descriptor of K step kt (zero-length past the end).
    __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rsrc(const char *ptr, int ld,
                                                                 uint32_t bytes, int kt, int nk)
    {
        const int k0 = kt * C::BK;
        const int64_t step = (KMAJ ? (int64_t)k0 : (int64_t)k0 * ld) * ES;   // bytes
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)(ptr + step), 0, kt < nk ? (int)(bytes - (uint32_t)step) : 0, kRsrcWord3);
    }

    // K tail of a k-major tile: this lane's chunk lies past K.
    __device__ __forceinline__ bool dead(int kt, int nk, int K) const
    {
        if constexpr (KMAJ && !C::WHOLE_K)
            return (kt == nk - 1) && (kc >= K - kt * C::BK);
        else
            return false;
    }
};

template <class C>
struct DirectLoader {
    using ACopy = OperandCopy<C, C::A_KMAJ, C::BM, C::A_LOADS>;
    using BCopy = OperandCopy<C, C::B_KMAJ, C::BN, C::B_LOADS>;
    // Per-instruction lane offsets are kept in registers when there are few
    // of them; otherwise they are rebuilt at issue from lane constants.
    static constexpr bool KEEP = C::LOADS <= 8;
    uint32_t voff[KEEP ? C::LOADS : 1];
    ACopy a;
    BCopy b;
    uint32_t lds0;     // LDS byte address of the workgroup's buffer

    __device__ __forceinline__ uint32_t a_off(const Params &p, int t, int m0) const
    {
        return a.off(t, m0, p.M, p.lda);
    }

    __device__ __forceinline__ uint32_t b_off(const Params &p, int t, int n0) const
    {
        return b.off(t, n0, p.N, p.ldb);
    }

    __device__ __forceinline__ void init(const Params &p, const char *smem, int m0, int n0)
    {
        a.init(m0, p.lda);
        b.init(n0, p.ldb);
        lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
        if constexpr (KEEP) {
#pragma unroll
            for (int t = 0; t < C::A_LOADS; t++)
                voff[t] = a_off(p, t, m0);
#pragma unroll
            for (int t = 0; t < C::B_LOADS; t++)
                voff[C::A_LOADS + t] = b_off(p, t, n0);
        }
    }

    // Issue copy instruction T (A copies first, then B) of K step kt into
    // LDS stage S.
    template <int S, int T>
    __device__ __forceinline__ void issue_one(const Params &p, int kt, int nk, int m0, int n0)
    {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if constexpr (T < C::A_LOADS) {
            const __amdgpu_buffer_rsrc_t ra = ACopy::rsrc((const char *)p.A, p.lda, p.a_bytes, kt, nk);
            const uint32_t o = KEEP ? voff[T] : a_off(p, T, m0);
            [[maybe_unused]] const uint32_t dst =
                lds0 + S * C::A_BYTES + (wave * C::A_LOADS + T) * 1024;
#ifdef TG_LDS_POISON
            poison16(dst + 16 * (threadIdx.x & 63));   // the bytes this lane's copy writes
            wait_lgkmcnt0();
#endif
            if constexpr (C::SCHED == 3)
                dma16_at<S * C::A_BYTES + T * 1024>(ra, o, lds0 + wave * C::A_LOADS * 1024);
            else
                dma16(ra, a.dead(kt, nk, p.K) ? kOOB : o, dst);
        } else {
            constexpr int t = T - C::A_LOADS;
            const __amdgpu_buffer_rsrc_t rb = BCopy::rsrc((const char *)p.B, p.ldb, p.b_bytes, kt, nk);
            const uint32_t o = KEEP ? voff[T] : b_off(p, t, n0);
            [[maybe_unused]] const uint32_t dst =
                lds0 + C::STAGES * C::A_BYTES + S * C::B_BYTES + (wave * C::B_LOADS + t) * 1024;
#ifdef TG_LDS_POISON
            poison16(dst + 16 * (threadIdx.x & 63));
            wait_lgkmcnt0();
#endif
            if constexpr (C::SCHED == 3)
                dma16_at<C::STAGES * C::A_BYTES + S * C::B_BYTES + t * 1024>(
                    rb, o, lds0 + wave * C::B_LOADS * 1024);
            else
                dma16(rb, b.dead(kt, nk, p.K) ? kOOB : o, dst);
        }
    }

    // Copy instructions [T0, T1) of K step kt into LDS stage S.
    template <int S, int T0 = 0, int T1 = C::LOADS>
    __device__ __forceinline__ void issue(const Params &p, int kt, int nk, int m0, int n0)
    {
        if constexpr (T0 < T1) {
            issue_one<S, T0>(p, kt, nk, m0, n0);
            issue<S, T0 + 1, T1>(p, kt, nk, m0, n0);
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
    int a_off[C::A_NOFF], b_off[C::B_NOFF];
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
                                              int m0, int n0)
{
    if constexpr (T < C::LOADS) {
        if constexpr (Spread<C>::pos(T) == OFF) {
            __builtin_amdgcn_sched_barrier(0);
            ld.template issue_one<(W + C::STAGES) % C::STAGES, T>(p, kt0 + W + C::STAGES, nk, m0, n0);
            __builtin_amdgcn_sched_barrier(0);
        }
        window_copies<C, W, OFF, T + 1>(p, ld, kt0, nk, m0, n0);
    }
}

// MFMAs [I, HI) of the k-step; MFMA I sits at position OFF of window W.
template <class C, int W, int OFF, int I, int HI>
__device__ __forceinline__ void mfma_window(const Params &p, DirectLoader<C> &ld, int kt0, int nk,
                                            int m0, int n0, const half8 (&fa)[C::MT],
                                            const half8 (&fb)[C::NT],
                                            typename C::acc_t (&acc)[C::MT][C::NT])
{
    if constexpr (I < HI) {
        constexpr int mt = I / C::NT, nt = I % C::NT;
        acc[mt][nt] = mfma<C>(fb[nt], fa[mt], acc[mt][nt]);
        window_copies<C, W, OFF>(p, ld, kt0, nk, m0, n0);
        mfma_window<C, W, OFF + 1, I + 1, HI>(p, ld, kt0, nk, m0, n0, fa, fb, acc);
    }
}

// Schedule 3: MFMAs [I, HI) of the k-step as mfma_window, with the fragment
// reads of k-step ksn of tiles (as, bs) placed between them: read r (the B
// blocks first, then the A blocks in row order, the order in which the next
// k-step's rows need them) after MFMA IB + (r + 1) RI - 1, each pinned to its
// place.  One wave per SIMD has no second wave to issue its reads while its
// MFMAs wait; issued in one burst they filled the LDS command FIFO.
template <class C, int W, int OFF, int I, int HI, int P, int IB, int RI>
__device__ __forceinline__ void mfma_window_rd(const Params &p, DirectLoader<C> &ld, int kt0,
                                               int nk, int m0, int n0, PipeState<C> &st,
                                               const char *as, const char *bs, int ksn)
{
    if constexpr (I < HI) {
        constexpr int mt = I / C::NT, nt = I % C::NT;
        st.acc[mt][nt] = mfma<C>(st.fb[P][nt], st.fa[P][mt], st.acc[mt][nt]);
        constexpr int q = I - IB + 1;
        if constexpr (q > 0 && q % RI == 0 && q / RI <= C::MT + C::NT) {
            constexpr int r = q / RI - 1;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (r < C::NT)
                st.fb[1 - P][r] = read_block<C, C::B_KMAJ, C::BN>(bs, ksn, st.b_off, r);
            else
                st.fa[1 - P][r - C::NT] =
                    read_block<C, C::A_KMAJ, C::BM>(as, ksn, st.a_off, r - C::NT);
            __builtin_amdgcn_sched_barrier(0);
        }
        window_copies<C, W, OFF>(p, ld, kt0, nk, m0, n0);
        mfma_window_rd<C, W, OFF + 1, I + 1, HI, P, IB, RI>(p, ld, kt0, nk, m0, n0, st, as, bs,
                                                            ksn);
    }
}

// LDS read instructions of one fragment block: 1 (k-major, ds_read_b128) or
// 2 (mn-major, two transpose reads).
template <class C, bool KMAJ>
constexpr int reads_per_block()
{
    return KMAJ ? 1 : 2;
}

// MFMAs of block row mt (all NT columns) of the current k-step.
template <class C, int MT_>
__device__ __forceinline__ void mfma_row(const half8 &fa, const half8 (&fb)[C::NT],
                                         typename C::acc_t (&acc)[C::MT][C::NT])
{
#pragma unroll
    for (int nt = 0; nt < C::NT; nt++)
        acc[MT_][nt] = mfma<C>(fb[nt], fa, acc[MT_][nt]);
}

// Rows [LO, HI) of the k-step: each row's MFMAs, then (REFILL) the A block
// of that row for k-step ks_next of tile `as`, read into the register the
// row has just finished with, and XB of the next k-step's B reads.
template <class C, int LO, int HI, bool REFILL, int XB>
__device__ __forceinline__ void roll_rows(PipeState<C> &st, int P, const char *as, int ks_next)
{
    if constexpr (LO < HI) {
        mfma_row<C, LO>(st.fa[0][LO], st.fb[P], st.acc);
        __builtin_amdgcn_sched_group_barrier(0x008, C::NT, 0);
        if constexpr (REFILL) {
            st.fa[0][LO] = read_block<C, C::A_KMAJ, C::BM>(as, ks_next, st.a_off, LO);
            __builtin_amdgcn_sched_group_barrier(0x100, reads_per_block<C, C::A_KMAJ>() + XB, 0);
        } else if constexpr (XB > 0) {
            __builtin_amdgcn_sched_group_barrier(0x100, XB, 0);
        }
        roll_rows<C, LO + 1, HI, REFILL, XB>(st, P, as, ks_next);
    }
}

// SCHED 2: the rows [HM, MT) that follow the barrier, row I of them first
// issuing its MFMAs (they use fragments read before the barrier), then two of
// the copies that refill the freed stage S, then reads of the next k-step:
// after the first row all B fragments, after each row one A block of rows
// [0, HM) (which could not be read before the barrier) and the refill of the
// row just finished.  Every wave passes the barrier at about the same time;
// issued in one burst ahead of the MFMAs (SCHED 0), these copies and reads
// queued behind one another in every wave at once and the matrix cores sat
// idle: on 8192^3 MFMA busy 67.7 % against 73.1 % here, and 3 % more
// TFLOP/s in alternating rounds (issuing the reads before the copies in each
// row gained 2 %; copies between single MFMAs spilled registers in the loop).
template <class C, int S, int SN, int P, int I = 0>
__device__ __forceinline__ void post_barrier_rows(const Params &p, DirectLoader<C> &ld,
                                                  const char *smem, int kt0, int nk, int m0,
                                                  int n0, PipeState<C> &st)
{
    constexpr int HM = C::MT / 2;
    constexpr int ROWS = C::MT - HM;
    if constexpr (I < ROWS) {
        constexpr int R = HM + I;
        constexpr int CPR = (C::LOADS + ROWS - 1) / ROWS;   // copies per row
        constexpr int T0 = I * CPR < C::LOADS ? I * CPR : C::LOADS;
        constexpr int T1 = (I + 1) * CPR < C::LOADS ? (I + 1) * CPR : C::LOADS;
        mfma_row<C, R>(st.fa[0][R], st.fb[P], st.acc);
        __builtin_amdgcn_sched_barrier(0);
        ld.template issue<S, T0, T1>(p, kt0 + S + C::STAGES, nk, m0, n0);
        if constexpr (I == 0)
            read_operand<C, C::B_KMAJ, C::BN>(b_stage<C, SN>(smem), 0, st.b_off, st.fb[1 - P]);
        if constexpr (I < HM)
            st.fa[0][I] = read_block<C, C::A_KMAJ, C::BM>(a_stage<C, SN>(smem), 0, st.a_off, I);
        st.fa[0][R] = read_block<C, C::A_KMAJ, C::BM>(a_stage<C, SN>(smem), 0, st.a_off, R);
        __builtin_amdgcn_sched_barrier(0);
        post_barrier_rows<C, S, SN, P, I + 1>(p, ld, smem, kt0, nk, m0, n0, st);
    }
}

// The k-step with rolling A fragments (C::ROLL).  B fragments stay double-
// buffered by k-step parity P (all of them are needed until the last row);
// A block row mt is re-read for the next k-step as soon as row mt's MFMAs
// are issued.  In the k-step that ends a stage, rows before the barrier
// cannot refill (the next stage is not published yet): their blocks are read
// right after it, with the next B fragments and the copies of the freed stage.
template <class C, int U, bool FINAL>
__device__ __forceinline__ void pipe_kstep_roll(const Params &p, DirectLoader<C> &ld,
                                                const char *smem, int kt0, int nk, int m0, int n0,
                                                PipeState<C> &st)
{
    constexpr int S = U / C::KS, ks = U % C::KS, P = U % 2;
    constexpr int HM = C::MT / 2;
    constexpr int BRD = C::NT * reads_per_block<C, C::B_KMAJ>();   // B read instructions
    constexpr bool BARRIER = ks + 1 == C::KS && (!FINAL || S + 1 < C::STAGES);
    static_assert(C::MT % 2 == 0 && BRD % HM == 0, "rolling rows");
    if constexpr (ks + 1 < C::KS) {
        // next k-step of the same stage: its B fragments spread over the
        // first half of the rows, each A block after its own row
        read_operand<C, C::B_KMAJ, C::BN>(b_stage<C, S>(smem), ks + 1, st.b_off, st.fb[1 - P]);
        roll_rows<C, 0, HM, true, BRD / HM>(st, P, a_stage<C, S>(smem), ks + 1);
        roll_rows<C, HM, C::MT, true, 0>(st, P, a_stage<C, S>(smem), ks + 1);
    } else if constexpr (BARRIER && C::SCHED == 2) {
        constexpr int SN = (S + 1) % C::STAGES;
        roll_rows<C, 0, HM, false, 0>(st, P, nullptr, 0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(C::STAGES - 2) * C::LOADS>();   // my copies of the next step landed
        lds_barrier();                               // everyone's did; stage S is free
        post_barrier_rows<C, S, SN, P>(p, ld, smem, kt0, nk, m0, n0, st);
    } else if constexpr (BARRIER) {
        constexpr int SN = (S + 1) % C::STAGES;
        roll_rows<C, 0, HM, false, 0>(st, P, nullptr, 0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(C::STAGES - 2) * C::LOADS>();   // my copies of the next step landed
        lds_barrier();                               // everyone's did; stage S is free
        read_operand<C, C::B_KMAJ, C::BN>(b_stage<C, SN>(smem), 0, st.b_off, st.fb[1 - P]);
#pragma unroll
        for (int mt = 0; mt < HM; mt++)
            st.fa[0][mt] = read_block<C, C::A_KMAJ, C::BM>(a_stage<C, SN>(smem), 0, st.a_off, mt);
        ld.template issue<S>(p, kt0 + S + C::STAGES, nk, m0, n0);
        __builtin_amdgcn_sched_barrier(0);
        roll_rows<C, HM, C::MT, true, 0>(st, P, a_stage<C, SN>(smem), 0);
    } else {
        roll_rows<C, 0, C::MT, false, 0>(st, P, nullptr, 0);
    }
}

// k-step U (0 .. STAGES*KS-1) of a loop body; FINAL: the body that ends the
// K loop (no barrier, reads or copies after its last k-step).
template <class C, int U, bool FINAL>
__device__ __forceinline__ void pipe_kstep(const Params &p, DirectLoader<C> &ld, const char *smem,
                                           int kt0, int nk, int m0, int n0, PipeState<C> &st)
{
    constexpr int S = U / C::KS, ks = U % C::KS, P = U % 2;
    constexpr int NMF = C::MT * C::NT;
    constexpr int NRD = C::MT + 2 * C::NT;
    constexpr int H = NMF / 2;
    constexpr int R = H / NRD > 0 ? H / NRD : 1;
    constexpr bool BARRIER = ks + 1 == C::KS && (!FINAL || S + 1 < C::STAGES);
    if constexpr (C::ROLL) {
        pipe_kstep_roll<C, U, FINAL>(p, ld, smem, kt0, nk, m0, n0, st);
    } else if constexpr (C::SCHED == 1 || C::SCHED == 3) {
        // position of this k-step's first MFMA in window S-1
        constexpr int OFF = H + ks * NMF;
        constexpr int NB = C::MT + C::NT;   // fragment blocks per k-step
        if constexpr (!BARRIER) {
            if constexpr (C::SCHED == 3 && ks + 1 < C::KS) {
                static_assert(NMF >= NB, "a read slot per block");
                mfma_window_rd<C, S - 1, OFF, 0, NMF, P, 0, NMF / NB>(
                    p, ld, kt0, nk, m0, n0, st, a_stage<C, S>(smem), b_stage<C, S>(smem), ks + 1);
            } else {
                if constexpr (ks + 1 < C::KS)
                    read_frags<C>(a_stage<C, S>(smem), b_stage<C, S>(smem), ks + 1, st.a_off,
                                  st.b_off, st.fa[1 - P], st.fb[1 - P]);
                mfma_window<C, S - 1, OFF, 0, NMF>(p, ld, kt0, nk, m0, n0, st.fa[P], st.fb[P],
                                                   st.acc);
            }
        } else {
            constexpr int SN = (S + 1) % C::STAGES;
            mfma_window<C, S - 1, OFF, 0, H>(p, ld, kt0, nk, m0, n0, st.fa[P], st.fb[P], st.acc);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<(C::STAGES - 2) * C::LOADS>();   // my copies of the next step landed
            lds_barrier();                               // everyone's did; stage S is free
            if constexpr (C::SCHED == 3) {
                // the next stage's first fragments between the rest of this
                // k-step's MFMAs
                static_assert(NMF - H >= NB, "a read slot per block");
                mfma_window_rd<C, S, 0, H, NMF, P, H, (NMF - H) / NB>(
                    p, ld, kt0, nk, m0, n0, st, a_stage<C, SN>(smem), b_stage<C, SN>(smem), 0);
            } else {
                read_frags<C>(a_stage<C, SN>(smem), b_stage<C, SN>(smem), 0, st.a_off, st.b_off,
                              st.fa[1 - P], st.fb[1 - P]);
                mfma_window<C, S, 0, H, NMF>(p, ld, kt0, nk, m0, n0, st.fa[P], st.fb[P], st.acc);
            }
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
        ld.template issue<S>(p, kt0 + S + C::STAGES, nk, m0, n0);
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
    if constexpr (C::SCHED == 1 || C::SCHED == 3) {
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
                                          int kt0, int nk, int m0, int n0, PipeState<C> &st)
{
    if constexpr (U < C::STAGES * C::KS) {
        pipe_kstep<C, U, FINAL>(p, ld, smem, kt0, nk, m0, n0, st);
        pipe_body<C, FINAL, U + 1>(p, ld, smem, kt0, nk, m0, n0, st);
    }
}

// Arguments of K slice z = blockIdx.y (split-K): A and B start at the
// slice's first K element, K is the slice's length, the buffer ranges end
// where the operand ends -- for an operand whose rows run along K (mn-major),
// after the slice's last K row, so that the copies of a partial last K step
// read zeros instead of the next slice's rows -- and C is the slice's own
// partial-product array.
template <class C>
__device__ __forceinline__ void k_slice(Params &p)
{
    const int z = blockIdx.y;
    const int k0 = z * p.k_split;
    const int kz = min(p.k_split, p.K - k0);
    const int64_t a_off = (C::A_KMAJ ? (int64_t)k0 : (int64_t)k0 * p.lda) * C::ES;
    const int64_t b_off = (C::B_KMAJ ? (int64_t)k0 : (int64_t)k0 * p.ldb) * C::ES;
    p.A = (const char *)p.A + a_off;
    p.B = (const char *)p.B + b_off;
    if (p.a_bytes) {
        uint32_t r = p.a_bytes - (uint32_t)a_off;
        if constexpr (!C::A_KMAJ)
            r = min(r, (uint32_t)(((int64_t)(kz - 1) * p.lda + p.M) * C::ES));
        p.a_bytes = r;
    }
    if (p.b_bytes) {
        uint32_t r = p.b_bytes - (uint32_t)b_off;
        if constexpr (!C::B_KMAJ)
            r = min(r, (uint32_t)(((int64_t)(kz - 1) * p.ldb + p.N) * C::ES));
        p.b_bytes = r;
    }
    p.K = kz;
    p.C = (char *)p.C + (int64_t)z * p.c_slice_bytes;
}

template <class C, typename OutT, bool BIAS, bool SPLIT>
__global__ void __launch_bounds__(C::THREADS, 1) gemm_pipe(Params p)
{
    if constexpr (SPLIT)
        k_slice<C>(p);
    static_assert((C::STAGES * C::KS) % 2 == 0, "register double buffer parity per loop body");
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
#ifdef TG_LDS_POISON
    poison_all<C::LDS_BYTES, C::THREADS>(smem);
#endif
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
        acc_fence<C, false>(st.acc);
        fragment_offsets<C>(wm, wn, st.a_off, st.b_off);
        DirectLoader<C> ld;
        ld.init(p, smem, m0, n0);
        if constexpr (C::SCHED == 1 || C::SCHED == 3) {
            // steps 0 .. STAGES-2 whole; of step STAGES-1 the copies whose
            // window position precedes the loop (the rest come from window -1
            // of the first loop body)
            [&]<int... S>(std::integer_sequence<int, S...>) {
                (ld.template issue<S>(p, S, nk, m0, n0), ...);
            }(std::make_integer_sequence<int, C::STAGES - 1>{});
            [&]<int... T>(std::integer_sequence<int, T...>) {
                ((Spread<C>::pos(T) < Spread<C>::H
                      ? ld.template issue_one<C::STAGES - 1, T>(p, C::STAGES - 1, nk, m0, n0)
                      : void()),
                 ...);
            }(std::make_integer_sequence<int, C::LOADS>{});
        } else {
            [&]<int... S>(std::integer_sequence<int, S...>) {
                (ld.template issue<S>(p, S, nk, m0, n0), ...);
            }(std::make_integer_sequence<int, C::STAGES>{});
        }
        wait_vmcnt<prologue_after_step0<C>()>();   // step 0 landed
        lds_barrier();
        read_frags<C>(a_stage<C, 0>(smem), b_stage<C, 0>(smem), 0, st.a_off, st.b_off, st.fa[0],
                      st.fb[0]);
        const int nsteps = (nk + C::STAGES - 1) / C::STAGES * C::STAGES;
        int kt = 0;
        for (; kt + C::STAGES < nsteps; kt += C::STAGES)
            pipe_body<C, false>(p, ld, smem, kt, nk, m0, n0, st);
        pipe_body<C, true>(p, ld, smem, kt, nk, m0, n0, st);
        // drain the dummy copies (they write zeros into LDS) and let every
        // wave finish its fragment reads before LDS is reused for the epilogue
        wait_vmcnt<0>();
        lds_barrier();
        acc_fence<C, true>(st.acc);
    }
    epilogue<C, OutT, BIAS>(p, smem, m0 + wm * C::TM, n0 + wn * C::TN, st.acc);
}

// ============================================================================
// General path: register-staged copies; any pointer alignment (2-byte) and any
// leading dimensions.  Every 16-byte chunk of a tile is one unaligned vector
// load (the memory system serves misaligned vector loads of global memory).
// A chunk that crosses the K or N edge, or lies past it, is still loaded as
// 16 bytes -- from a place inside the operand's footprint, see src() -- and
// the elements outside the matrix are cleared when the chunk is written to
// LDS, after its data has arrived anyway.  So the loads of a K step never
// wait on each other, and edge tiles pipeline like interior ones.  Same LDS
// layout and fragment reads as the direct path, two LDS stages.
// ============================================================================
// One operand's share of a K step, register-staged.  Chunk t of this thread
// sits at the same LDS position as the direct copies would put it; offsets
// are in elements from the tile corner (x0, k0) of a k-major operand or
// (k0, x0) of an mn-major one, where x runs along M (A) or N (B).  The
// operand's footprint is the element range [0, (rows - 1) ld + cols) of its
// stored rows; every element of it is readable.
template <class C, bool KMAJ, int R, int NLOADS>
struct OperandStage {
    static constexpr int ES = C::ES;
    static constexpr int CE = 16 / ES;                               // elements per chunk
    static constexpr int RCH = KMAJ ? C::KROWB / 16 : R * ES / 16;   // chunks per row
    static constexpr int RPL = 64 / RCH;

    // row (along x, k-major) or k-row (mn-major) of chunk t, and its
    // logical column in elements (k, k-major; x, mn-major)
    __device__ __forceinline__ static int row(int t)
    {
        const int lane = threadIdx.x & 63;
        return ((threadIdx.x >> 6) * NLOADS + t) * RPL + lane / RCH;
    }
    __device__ __forceinline__ static int col(int t)
    {
        const int lane = threadIdx.x & 63;
        if constexpr (KMAJ)
            return ((lane % RCH) ^ swz_a<C::KROWB>(row(t))) * CE;
        else
            return ((lane % RCH) ^ swz_mn<ES, R>(row(t))) * CE;
    }
    __device__ __forceinline__ static uint32_t off(int t, int ld)
    {
        return (uint32_t)(row(t) * ld + col(t));
    }

    // Stored rows of the tile inside the matrix, and elements of a tile row
    // inside it, for the tile at (x0, k0) of an operand with X rows along x.
    __device__ __forceinline__ static int rows_in(int x0, int X, int k0, int K)
    {
        return KMAJ ? X - x0 : K - k0;
    }
    __device__ __forceinline__ static int cols_in(int x0, int X, int k0, int K)
    {
        return KMAJ ? K - k0 : X - x0;
    }
    // Elements of chunk t inside the matrix, from its first: 0 .. CE.
    __device__ __forceinline__ static int valid(int t, int rin, int cin)
    {
        return row(t) < rin ? min(max(cin - col(t), 0), CE) : 0;
    }
    // Footprint in elements, or 0 when it cannot serve the 16-byte loads:
    // fewer than CE elements in all, or rows shorter than a chunk (then a
    // partial chunk of any row may end past the footprint).
    __device__ __forceinline__ static int64_t footprint(int X, int K, int ld)
    {
        const int rows = KMAJ ? X : K, cols = KMAJ ? K : X;
        const int64_t f = (int64_t)(rows - 1) * ld + cols;
        return (ld < CE || f < CE) ? 0 : f;
    }

    // Element index of the 16 bytes loaded for chunk t (footprint >= CE):
    //  - a chunk with all CE elements inside the matrix: the chunk itself;
    //  - a partial chunk of any row but the matrix's last: the chunk itself,
    //    whose tail past the row end is padding or the next row, inside the
    //    footprint since rows are at least CE long;
    //  - the partial chunk of the last row, which would end past the
    //    footprint: the CE elements ending at the footprint's end, i.e. the
    //    chunk moved back by CE - n elements (undone at the LDS write);
    //  - a chunk wholly outside the matrix: element 0 (any readable place;
    //    its data is replaced by zeros at the LDS write).
    __device__ __forceinline__ static int64_t src(int t, int64_t corner, uint32_t o, int rin,
                                                  int cin)
    {
        const int n = valid(t, rin, cin);
        int64_t e = corner + o;
        if (n < CE && row(t) == rin - 1)
            e -= CE - n;
        return n == 0 ? 0 : e;
    }

    // The chunk's elements as they go to LDS: moved forward again for the
    // last row's partial chunk, and zeros past the matrix edge.
    __device__ __forceinline__ static half8 fix(half8 v, int t, int rin, int cin)
    {
        const int n = valid(t, rin, cin);
        if (n < CE) {   // partial or outside: rare, skipped when no lane has one
            uint32_t w[4];
            __builtin_memcpy(w, &v, 16);
            if (n > 0 && row(t) == rin - 1) {
                // the loaded bytes start (CE - n) elements early: shift the
                // 16 bytes down by that many (q dwords and b bytes)
                const int sb = (CE - n) * ES, q = sb >> 2, b = sb & 3;
                uint32_t x[5];
#pragma unroll
                for (int i = 0; i < 5; i++) {
                    uint32_t y = 0;
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        y = (i + j < 4 && q == j) ? w[i + j] : y;
                    x[i] = y;
                }
#pragma unroll
                for (int i = 0; i < 4; i++)
                    w[i] = __builtin_amdgcn_alignbyte(x[i + 1], x[i], b);
            }
            const int keep = n * ES;   // bytes of the chunk inside the matrix
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int kb = keep - 4 * i;
                w[i] = kb >= 4 ? w[i] : (kb <= 0 ? 0u : w[i] & ((1u << (8 * kb)) - 1u));
            }
            __builtin_memcpy(&v, w, 16);
        }
        return v;
    }

    // Element-by-element load of chunk t with zeros past the edge: taken by
    // both operands when either one's footprint cannot serve 16-byte loads
    // (under CE elements, or rows shorter than a chunk).
    __device__ __forceinline__ static half8 load_small(const char *ptr, uint32_t o, int t,
                                                       int64_t corner, int rin, int cin)
    {
        half8 v = {};
        const int n = valid(t, rin, cin);
        const char *src = ptr + (corner + o) * ES;
        char *d = (char *)&v;
#pragma unroll
        for (int e = 0; e < CE; e++)
            if (e < n)
                __builtin_memcpy(d + e * ES, src + e * ES, ES);
        return v;
    }
};

template <class C>
struct StagedLoader {
    using AS = OperandStage<C, C::A_KMAJ, C::BM, C::A_LOADS>;
    using BS = OperandStage<C, C::B_KMAJ, C::BN, C::B_LOADS>;
    half8 r[C::LOADS];       // one K step of this thread's chunks: A first, then B
    uint32_t off[C::LOADS];  // element offset of each chunk from the tile corner
                             // (host: in-tile offsets stay below 2^31)
    bool small;              // an operand's footprint is too small for 16-byte
                             // loads (uniform)

    __device__ __forceinline__ void init(const Params &p)
    {
#pragma unroll
        for (int t = 0; t < C::A_LOADS; t++)
            off[t] = AS::off(t, p.lda);
#pragma unroll
        for (int t = 0; t < C::B_LOADS; t++)
            off[C::A_LOADS + t] = BS::off(t, p.ldb);
        small = AS::footprint(p.M, p.K, p.lda) == 0 || BS::footprint(p.N, p.K, p.ldb) == 0;
    }

    __device__ __forceinline__ static bool interior(const Params &p, int m0, int n0, int kt)
    {
        return m0 + C::BM <= p.M && n0 + C::BN <= p.N && (kt + 1) * C::BK <= p.K;
    }
    __device__ __forceinline__ static int64_t a_corner(const Params &p, int m0, int k0)
    {
        return C::A_KMAJ ? (int64_t)m0 * p.lda + k0 : (int64_t)k0 * p.lda + m0;
    }
    __device__ __forceinline__ static int64_t b_corner(const Params &p, int n0, int k0)
    {
        return C::B_KMAJ ? (int64_t)n0 * p.ldb + k0 : (int64_t)k0 * p.ldb + n0;
    }

    // Load K step kt into registers: one 16-byte load per chunk, issued
    // back to back; the LDS write clears what lies outside the matrix (so
    // steps past the end write zeros).  Three exclusive paths: interior
    // tiles, edge tiles, and (tiny operands only) element-by-element loads
    // that finish before the path ends, so that no load of that path is
    // still counted where the paths join and the loads of the other two
    // paths never wait for one another.
    __device__ __forceinline__ void load(const Params &p, int m0, int n0, int kt)
    {
        const int k0 = kt * C::BK;
        const char *pa = (const char *)p.A, *pb = (const char *)p.B;
        const int64_t ca = a_corner(p, m0, k0), cb = b_corner(p, n0, k0);
        if (interior(p, m0, n0, kt)) {
#pragma unroll
            for (int t = 0; t < C::LOADS; t++)
                __builtin_memcpy(&r[t], t < C::A_LOADS ? pa + (ca + off[t]) * C::ES
                                                       : pb + (cb + off[t]) * C::ES, 16);
            return;
        }
        const int ra = AS::rows_in(m0, p.M, k0, p.K), qa = AS::cols_in(m0, p.M, k0, p.K);
        const int rb = BS::rows_in(n0, p.N, k0, p.K), qb = BS::cols_in(n0, p.N, k0, p.K);
        if (!small) {
            int64_t e[C::LOADS];
#pragma unroll
            for (int t = 0; t < C::A_LOADS; t++)
                e[t] = AS::src(t, ca, off[t], ra, qa);
#pragma unroll
            for (int t = 0; t < C::B_LOADS; t++)
                e[C::A_LOADS + t] = BS::src(t, cb, off[C::A_LOADS + t], rb, qb);
#pragma unroll
            for (int t = 0; t < C::LOADS; t++)
                __builtin_memcpy(&r[t], (t < C::A_LOADS ? pa : pb) + e[t] * C::ES, 16);
        } else {
#pragma unroll
            for (int t = 0; t < C::A_LOADS; t++)
                r[t] = AS::load_small(pa, off[t], t, ca, ra, qa);
#pragma unroll
            for (int t = 0; t < C::B_LOADS; t++)
                r[C::A_LOADS + t] = BS::load_small(pb, off[C::A_LOADS + t], t, cb, rb, qb);
            wait_vmcnt<0>();
        }
    }

    // Registers of K step kt -> LDS stage S, in the layout the direct copies
    // produce; chunks of an edge step are first put right (fix()).
    template <int S>
    __device__ __forceinline__ void store(const Params &p, char *smem, int m0, int n0,
                                          int kt) const
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const bool edge = !interior(p, m0, n0, kt);
#ifdef TG_LDS_POISON
        // the stage's bytes this thread writes below, first as NaN
        {
            const uint32_t base =
                (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
#pragma unroll
            for (int t = 0; t < C::A_LOADS; t++)
                poison16(base + S * C::A_BYTES + (wave * C::A_LOADS + t) * 1024 + lane * 16);
#pragma unroll
            for (int t = 0; t < C::B_LOADS; t++)
                poison16(base + C::STAGES * C::A_BYTES + S * C::B_BYTES +
                         (wave * C::B_LOADS + t) * 1024 + lane * 16);
            wait_lgkmcnt0();
        }
#endif
        const int k0 = kt * C::BK;
        const int ra = AS::rows_in(m0, p.M, k0, p.K), qa = AS::cols_in(m0, p.M, k0, p.K);
        const int rb = BS::rows_in(n0, p.N, k0, p.K), qb = BS::cols_in(n0, p.N, k0, p.K);
#pragma unroll
        for (int t = 0; t < C::A_LOADS; t++) {
            half8 v = r[t];
            if (edge && !small)
                v = AS::fix(v, t, ra, qa);
            *(half8 *)(smem + S * C::A_BYTES + (wave * C::A_LOADS + t) * 1024 + lane * 16) = v;
        }
#pragma unroll
        for (int t = 0; t < C::B_LOADS; t++) {
            half8 v = r[C::A_LOADS + t];
            if (edge && !small)
                v = BS::fix(v, t, rb, qb);
            *(half8 *)(smem + C::STAGES * C::A_BYTES + S * C::B_BYTES +
                       (wave * C::B_LOADS + t) * 1024 + lane * 16) = v;
        }
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
        ld.template store<SN>(p, smem, m0, n0, kt0 + S + 1);   // its stage is free
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

template <class C, typename OutT, bool BIAS, bool SPLIT>
__global__ void __launch_bounds__(C::THREADS, 1) gemm_staged(Params p)
{
    if constexpr (SPLIT)
        k_slice<C>(p);
    static_assert(C::STAGES == 2, "the register-staged path double-buffers LDS");
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
#ifdef TG_LDS_POISON
    poison_all<C::LDS_BYTES, C::THREADS>(smem);
#endif
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
        ld.template store<0>(p, smem, m0, n0, 0);
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

// ============================================================================
// Single-stage reference kernel: one LDS buffer and no overlap of copies with
// compute.  Every K step: the register-staged loads of the step (any
// alignment, as above), a barrier (every wave is past its last fragment read
// of the previous step), the LDS writes, a barrier, then the step's k-steps,
// each reading its fragments and issuing its MFMAs in turn.  The plainest
// schedule of the tiled product: the pipelined kernels are checked against it
// bit for bit on integer inputs.
// ============================================================================
template <class C, typename OutT, bool BIAS, bool SPLIT>
__global__ void __launch_bounds__(C::THREADS, 1) gemm_single(Params p)
{
    if constexpr (SPLIT)
        k_slice<C>(p);
    static_assert(C::STAGES == 1, "one LDS stage");
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
#ifdef TG_LDS_POISON
    poison_all<C::LDS_BYTES, C::THREADS>(smem);
#endif
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
        for (int kt = 0; kt < nk; kt++) {
            ld.load(p, m0, n0, kt);
            lds_barrier();   // every wave is past the previous step's reads
            ld.template store<0>(p, smem, m0, n0, kt);
            lds_barrier();   // the step is in LDS
#pragma unroll
            for (int ks = 0; ks < C::KS; ks++) {
                read_frags<C>(a_stage<C, 0>(smem), b_stage<C, 0>(smem), ks, st.a_off, st.b_off,
                              st.fa[0], st.fb[0]);
                mfma_range<C, 0, C::MT * C::NT>(st.fa[0], st.fb[0], st.acc);
            }
        }
        lds_barrier();   // every wave past its last fragment read
    }
    epilogue<C, OutT, BIAS>(p, smem, m0 + wm * C::TM, n0 + wn * C::TN, st.acc);
}

// ------------------------------------------------------------ instances --
template <class C, int TA, int TB>
using WithOps = Cfg<C::BM, C::BN, C::BK, C::WAVES_M, C::WAVES_N, C::STAGES, C::MI, C::SCHED, TA, TB,
                    C::ES>;

template <class C, int KIND>
hipError_t launch_ops(const Params &p, bool f16_out, bool bias, hipStream_t s)
{
    const dim3 grid(p.tiles_m * p.tiles_n, p.splits > 1 ? p.splits : 1), block(C::THREADS);
#define TG_GO(KERNEL, OUT, B, SPLIT)                                                 \
    do {                                                                             \
        hipLaunchKernelGGL((KERNEL<C, OUT, B, SPLIT>), grid, block, 0, s, p);        \
        return hipGetLastError();                                                    \
    } while (0)
#define TG_KIND(OUT, B, SPLIT)                                                       \
    do {                                                                             \
        if constexpr (KIND == 2)                                                     \
            TG_GO(gemm_pipe, OUT, B, SPLIT);                                         \
        else if constexpr (KIND == 1)                                                \
            TG_GO(gemm_single, OUT, B, SPLIT);                                       \
        else                                                                         \
            TG_GO(gemm_staged, OUT, B, SPLIT);                                       \
    } while (0)
    if (p.splits > 1) {   // K slices: fp32 (int32) partial products, no bias
        if (f16_out || bias)
            return hipErrorInvalidValue;
        using PartT = std::conditional_t<C::ES == 1, int32_t, float>;
        TG_KIND(PartT, false, true);
    }
    if constexpr (C::ES == 1) {   // int8 operands: int32 C, no bias
        if (f16_out || bias)
            return hipErrorInvalidValue;
        TG_KIND(int32_t, false, false);
    } else {
        if (f16_out) { if (bias) TG_KIND(_Float16, true, false); else TG_KIND(_Float16, false, false); }
        else { if (bias) TG_KIND(float, true, false); else TG_KIND(float, false, false); }
    }
#undef TG_KIND
#undef TG_GO
}

// OPS: bit (1 << (2 TA + TB)) set for each operand orientation instantiated.
template <class C, int KIND, int OPS>
hipError_t launch_cfg(const Params &p, bool f16_out, bool bias, hipStream_t s)
{
    const int op = 2 * p.trans_a + p.trans_b;
    if constexpr ((OPS & 1) != 0)
        if (op == 0) return launch_ops<WithOps<C, 0, 0>, KIND>(p, f16_out, bias, s);
    if constexpr ((OPS & 2) != 0)
        if (op == 1) return launch_ops<WithOps<C, 0, 1>, KIND>(p, f16_out, bias, s);
    if constexpr ((OPS & 4) != 0)
        if (op == 2) return launch_ops<WithOps<C, 1, 0>, KIND>(p, f16_out, bias, s);
    if constexpr ((OPS & 8) != 0)
        if (op == 3) return launch_ops<WithOps<C, 1, 1>, KIND>(p, f16_out, bias, s);
    return hipErrorInvalidValue;
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

template <int ID, class CFG, int KIND, int OPS>
LaunchFn shard_launch()
{
    if constexpr (ID % TG_SHARDS == TG_SHARD)
        return &launch_cfg<CFG, KIND, OPS>;
    else
        return nullptr;
}

// ------------------------------------------------------ split-K reduction --
// One lane per 4 consecutive columns of a row: the slices' partials are
// summed in slice order (fp32, or int32 for int8 operands: exact), then the
// bias is added and ReLU applied, and the result converted to C's type.
// Memory-bound: 16-byte loads of each slice and one store of C per lane,
// consecutive lanes on consecutive columns.
template <typename AccT, typename OutT, bool BIAS>
__global__ void __launch_bounds__(256) splitk_reduce(ReduceParams r)
{
    const int64_t per_row = (r.N + 3) / 4;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= (int64_t)r.M * per_row)
        return;
    const int64_t row = g / per_row;
    const int col = (int)(g - row * per_row) * 4;
    const AccT *src = (const AccT *)r.ws + row * r.N + col;
    AccT v[4];
    if (r.vec_ws && col + 3 < r.N) {
        using V4 = std::conditional_t<std::is_same_v<AccT, int32_t>, int4v, float4v>;
        V4 a = *(const V4 *)src;
        for (int z = 1; z < r.splits; z++) {
            const V4 b = *(const V4 *)(src + z * r.slice_elems);
            a += b;
        }
#pragma unroll
        for (int j = 0; j < 4; j++)
            v[j] = a[j];
    } else {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[j] = 0;
            if (col + j < r.N) {
                v[j] = src[j];
                for (int z = 1; z < r.splits; z++)
                    v[j] += src[z * r.slice_elems + j];
            }
        }
    }
    OutT o[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if constexpr (BIAS) {
            const float x = (float)v[j] + (col + j < r.N ? r.bias[col + j] : 0.f);
            o[j] = (OutT)(x > 0.f ? x : 0.f);
        } else {
            o[j] = (OutT)v[j];
        }
    }
    OutT *dst = (OutT *)r.C + row * r.ldc + col;
    if (r.vec_c && col + 3 < r.N) {
        if constexpr (sizeof(OutT) == 2) {
            typedef _Float16 h4 __attribute__((ext_vector_type(4)));
            *(h4 *)dst = h4{o[0], o[1], o[2], o[3]};
        } else {
            typedef OutT o4 __attribute__((ext_vector_type(4)));
            *(o4 *)dst = o4{o[0], o[1], o[2], o[3]};
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; j++)
            if (col + j < r.N)
                dst[j] = o[j];
    }
}

#if TG_SHARD == 0
hipError_t launch_splitk_reduce(const ReduceParams &r, OutKind out, hipStream_t s)
{
    const int64_t lanes = (int64_t)r.M * ((r.N + 3) / 4);
    if (lanes <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
    const bool b = r.bias != nullptr;
    if (out == kOutI32) {
        if (b)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((splitk_reduce<int32_t, int32_t, false>), grid, block, 0, s, r);
    } else if (out == kOutF16) {
        if (b)
            hipLaunchKernelGGL((splitk_reduce<float, _Float16, true>), grid, block, 0, s, r);
        else
            hipLaunchKernelGGL((splitk_reduce<float, _Float16, false>), grid, block, 0, s, r);
    } else {
        if (b)
            hipLaunchKernelGGL((splitk_reduce<float, float, true>), grid, block, 0, s, r);
        else
            hipLaunchKernelGGL((splitk_reduce<float, float, false>), grid, block, 0, s, r);
    }
    return hipGetLastError();
}
#endif

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

#define TG_CONFIG_ROW(ID, BM, BN, BK, WM, WN, ST, MI, KIND, SCH, OPS, ES)                          \
    shard_launch<ID, Cfg<BM, BN, BK, WM, WN, ST, MI, SCH, 0, 0, ES>, KIND, OPS>(),
const LaunchFn TG_CAT(kShardLaunch, TG_SHARD)[] = {
#include "tg_config_list.inc"
};
#undef TG_CONFIG_ROW
#else
// device pass: instantiate the kernels of this shard
#define TG_CONFIG_ROW(ID, BM, BN, BK, WM, WN, ST, MI, KIND, SCH, OPS, ES)                          \
    template LaunchFn shard_launch<ID, Cfg<BM, BN, BK, WM, WN, ST, MI, SCH, 0, 0, ES>, KIND, OPS>();
#include "tg_config_list.inc"
#undef TG_CONFIG_ROW
#endif

#if TG_SHARD == 0 && !defined(__HIP_DEVICE_COMPILE__)
#define TG_CONFIG_ROW(ID, BM, BN, BK, WM, WN, ST, MI, KIND, SCH, OPS, ES)                          \
    {ID, BM, BN, BK, ST, WM, WN, MI, (KIND) == 2,                                    \
     Cfg<BM, BN, BK, WM, WN, ST, MI, SCH, 0, 0, ES>::LDS_BYTES, OPS, ES,                   \
     Cfg<BM, BN, BK, WM, WN, ST, MI, SCH, 0, 0, ES>::WHOLE_K,                              \
     (KIND == 2 ? (ES == 1 ? "i8_pipe_" #BM "x" #BN "x" #BK "_s" #ST "_w" #WM "x" #WN "_mi" #MI \
                             "_c" #SCH                                                     \
                           : "pipe_" #BM "x" #BN "x" #BK "_s" #ST "_w" #WM "x" #WN "_mi" #MI   \
                             "_c" #SCH)                                                    \
     : KIND == 1 ? (ES == 1 ? "i8_single_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_mi" #MI \
                            : "single_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_mi" #MI)    \
                : (ES == 1 ? "i8_staged_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_mi" #MI   \
                           : "staged_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_mi" #MI))},

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
