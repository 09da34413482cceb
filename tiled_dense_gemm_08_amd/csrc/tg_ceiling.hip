// tg_ceiling.hip — the matrix cores' sustained fp16 (or int8) rate on given
// operand values, with no memory traffic in the timed loop.
//
// Workgroups of 8 waves, two per SIMD, as in the large GEMM kernels: every
// wave keeps a 128 x 64 accumulator tile (fp32, or int32 for int8) and two
// sets of operand fragments in registers, read once from the caller's buffer,
// and alternates between the two sets at every k-step, so the multiplier
// inputs change from one MFMA to the next as they do in a GEMM.  (With one
// wave per SIMD the 16x16 shapes keep the matrix core only about 80 % busy
// even on zero operands; two waves fill it.)  The rate this reaches is a
// property of the chip and of the operand values: under the board's power
// limit the shader clock drops when the operand bits toggle, so random
// operands run the matrix cores below the nominal dense peak, while all-zero
// ones reach it.  A GEMM on the same values with these MFMA shapes cannot
// exceed this rate; the bench reports its throughput against it.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tg_ceiling.h"

namespace tg {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;   // 8 waves, two per SIMD

// One k-step on every accumulator block: set s's A fragments (rows) against
// its B fragments (columns).  MI 16: 16x16x32 fp16 (k-step 32), 32: 32x32x16
// fp16 (one 16-deep slab per set, two sets = k-step 32), 64: 16x16x64 int8.
template <int MI, int NBM, int NBN, typename Acc>
__device__ __forceinline__ void kstep(const half8 (&a)[NBM], const half8 (&b)[NBN],
                                      Acc (&acc)[NBM][NBN])
{
#pragma unroll
    for (int i = 0; i < NBM; i++)
#pragma unroll
        for (int j = 0; j < NBN; j++) {
            if constexpr (MI == 64)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    __builtin_bit_cast(int4v, b[j]), __builtin_bit_cast(int4v, a[i]), acc[i][j],
                    0, 0, 0);
            else if constexpr (MI == 32)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a[i], acc[i][j], 0, 0, 0);
            else
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j], a[i], acc[i][j], 0, 0, 0);
        }
}

// Thread t's fragments of set s: A block j at chunk (16 t + 8 s + j) mod 4096
// of the buffer's first half, B block j at chunk 4096 + (8 t + 4 s + j) mod
// 4096 of its second half (16-byte chunks).
template <int MI>
__global__ void __launch_bounds__(kThreads, 1)
    mfma_ceiling_kernel(const half8 *__restrict__ in, float *__restrict__ sink, int iters)
{
    constexpr int BLK = MI == 32 ? 32 : 16;
    constexpr int NBM = 128 / BLK, NBN = 64 / BLK;   // accumulator blocks per wave
    using Acc = typename std::conditional<MI == 64, int4v,
                                          typename std::conditional<MI == 32, float16v,
                                                                    float4v>::type>::type;
    const int t = threadIdx.x;
    half8 a[2][NBM], b[2][NBN];
#pragma unroll
    for (int s = 0; s < 2; s++) {
#pragma unroll
        for (int j = 0; j < NBM; j++)
            a[s][j] = in[(16 * t + 8 * s + j) & 4095];
#pragma unroll
        for (int j = 0; j < NBN; j++)
            b[s][j] = in[4096 + ((8 * t + 4 * s + j) & 4095)];
    }
    Acc acc[NBM][NBN];
#pragma unroll
    for (int i = 0; i < NBM; i++)
#pragma unroll
        for (int j = 0; j < NBN; j++)
            acc[i][j] = Acc{};
    // two k-steps per trip (iters is even), the sets alternating; for MI 32 a
    // k-step of 32 is the two sets' 16-deep slabs
    for (int it = 0; it < iters; it += 2) {
        if constexpr (MI == 32) {
#pragma unroll
            for (int r = 0; r < 2; r++) {
                kstep<MI>(a[0], b[0], acc);
                kstep<MI>(a[1], b[1], acc);
            }
        } else {
            kstep<MI>(a[0], b[0], acc);
            kstep<MI>(a[1], b[1], acc);
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NBM; i++)
#pragma unroll
        for (int j = 0; j < NBN; j++)
#pragma unroll
            for (int r = 0; r < (int)(sizeof(Acc) / 4); r++)
                sum += (float)acc[i][j][r];
    sink[(int64_t)blockIdx.x * kThreads + t] = sum;
}

}  // namespace

hipError_t launch_mfma_ceiling(int mfma, const void *operands, float *sink, int iters,
                               int workgroups, hipStream_t s)
{
    const half8 *in = (const half8 *)operands;
    if (mfma == 32)
        mfma_ceiling_kernel<32><<<workgroups, kThreads, 0, s>>>(in, sink, iters);
    else if (mfma == 64)
        mfma_ceiling_kernel<64><<<workgroups, kThreads, 0, s>>>(in, sink, iters);
    else
        mfma_ceiling_kernel<16><<<workgroups, kThreads, 0, s>>>(in, sink, iters);
    return hipGetLastError();
}

}  // namespace tg
