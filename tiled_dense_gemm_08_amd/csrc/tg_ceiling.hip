// tg_ceiling.hip — the matrix cores' sustained fp16 rate on given operand
// values, with no memory traffic in the timed loop.
//
// Every wave keeps a 128 x 128 fp32 accumulator tile and two sets of operand
// fragments in registers, read once from the caller's buffer, and alternates
// between the two sets at every k-step of 32, so the multiplier inputs change
// from one MFMA to the next as they do in a GEMM.  The rate this reaches is a
// property of the chip and of the operand values: under the board's power
// limit the shader clock drops when the operand bits toggle, so random
// operands run the matrix cores well below the nominal dense peak, while
// all-zero ones reach it.  A GEMM on the same values cannot exceed this rate;
// the bench reports its throughput against both.
#include <hip/hip_runtime.h>

#include "tg_ceiling.h"

namespace tg {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;   // 4 waves, one per SIMD

// Thread t's fragments: chunks t * 32 .. t * 32 + 31 of the operand buffer
// (16 bytes each): set s, A block j at chunk 16 s + j, B block j at 16 s + 8 + j.
template <int MI>
__global__ void __launch_bounds__(kThreads, 1)
    mfma_ceiling_kernel(const half8 *__restrict__ in, float *__restrict__ sink, int iters)
{
    const int t = threadIdx.x;
    constexpr int NB = MI == 32 ? 4 : 8;   // MFMA blocks along each edge of 128
    half8 a[2][NB], b[2][NB];
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
        for (int j = 0; j < NB; j++) {
            a[s][j] = in[t * 32 + s * 16 + j];
            b[s][j] = in[t * 32 + s * 16 + 8 + j];
        }
    float sum = 0.0f;
    if constexpr (MI == 32) {
        float16v acc[NB][NB];
#pragma unroll
        for (int i = 0; i < NB; i++)
#pragma unroll
            for (int j = 0; j < NB; j++)
                acc[i][j] = float16v{};
        // one k-step of 32 = two 32x32x16 MFMAs per block, one per operand set
        for (int it = 0; it < iters; it++) {
#pragma unroll
            for (int s = 0; s < 2; s++)
#pragma unroll
                for (int i = 0; i < NB; i++)
#pragma unroll
                    for (int j = 0; j < NB; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[s][j], a[s][i],
                                                                           acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NB; i++)
#pragma unroll
            for (int j = 0; j < NB; j++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    sum += acc[i][j][r];
    } else {
        float4v acc[NB][NB];
#pragma unroll
        for (int i = 0; i < NB; i++)
#pragma unroll
            for (int j = 0; j < NB; j++)
                acc[i][j] = float4v{};
        // one k-step of 32 = one 16x16x32 MFMA per block; sets alternate per
        // k-step, two k-steps per trip (iters is even)
        for (int it = 0; it < iters; it += 2) {
#pragma unroll
            for (int s = 0; s < 2; s++)
#pragma unroll
                for (int i = 0; i < NB; i++)
#pragma unroll
                    for (int j = 0; j < NB; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[s][j], a[s][i],
                                                                           acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NB; i++)
#pragma unroll
            for (int j = 0; j < NB; j++)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    sum += acc[i][j][r];
    }
    sink[(int64_t)blockIdx.x * kThreads + t] = sum;
}

}  // namespace

hipError_t launch_mfma_ceiling(int mfma, const void *operands, float *sink, int iters,
                               int workgroups, hipStream_t s)
{
    const half8 *in = (const half8 *)operands;
    if (mfma == 32)
        mfma_ceiling_kernel<32><<<workgroups, kThreads, 0, s>>>(in, sink, iters);
    else
        mfma_ceiling_kernel<16><<<workgroups, kThreads, 0, s>>>(in, sink, iters);
    return hipGetLastError();
}

}  // namespace tg
