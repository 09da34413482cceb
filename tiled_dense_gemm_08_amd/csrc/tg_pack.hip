// tg_pack.hip — copy of a GEMM operand into the layout the direct global->LDS
// copies need: rows padded with zeros to a multiple of 16 bytes, the copy's
// leading dimension equal to that padded length, and a 16-byte aligned base.
// The dispatcher uses it for operands whose leading dimension, row length or
// base alignment rule the direct copies out, when the copy plus the direct
// kernel is predicted to beat the register-staged kernel.  Memory-bound: a
// thread moves 16-byte chunks of the copy, each read with one 16-byte load
// (any alignment of the element size) and written aligned.
#include <hip/hip_runtime.h>

#include "tg_pack.h"

namespace tg {

namespace {

struct PackArgs {
    PackOperand op[2];
    uint32_t chunks[2];   // 16-byte chunks of each packed copy
    uint32_t cpr[2];      // chunks per packed row
};

// Chunk c of the copies (the first copy's chunks first): where it goes, where
// its 16 bytes are read, and how many of its bytes lie inside the source row
// (`keep`, 0..16).  A chunk wholly inside the row is read in place.  The
// row's last, partial chunk is read as the 16 bytes that end at the row's
// end (rows of at least 16 bytes only) and shifted down by 16 - keep bytes
// afterwards; a chunk past the row's end reads the row's first 16 bytes and
// keeps none of them.  Every read stays inside the row.
struct ChunkRef {
    const char *src;
    char *dst;
    int keep;
    bool shifted;
};

__device__ __forceinline__ ChunkRef chunk_ref(const PackArgs &a, uint32_t c)
{
    const int w = c >= a.chunks[0];
    const PackOperand &p = a.op[w];
    const uint32_t q = w ? c - a.chunks[0] : c;
    const uint32_t r = q / a.cpr[w];
    const int64_t b = (int64_t)(q - r * a.cpr[w]) * 16;   // first byte of the chunk in its row
    const int64_t row_bytes = p.cols * p.es;
    const int64_t left = row_bytes - b;                    // row bytes from the chunk on
    const char *row = (const char *)p.src + (int64_t)r * p.ld * p.es;
    ChunkRef ref;
    ref.dst = (char *)p.dst + (int64_t)q * 16;
    ref.keep = left >= 16 ? 16 : (left > 0 ? (int)left : 0);
    ref.shifted = left > 0 && left < 16;
    ref.src = left >= 16 ? row + b : (left > 0 ? row + row_bytes - 16 : row);
    return ref;
}

// The chunk's bytes as they go to the copy: moved down by 16 - keep bytes
// when read shifted, and zeros from byte `keep` on.
__device__ __forceinline__ void finish_chunk(uint32_t (&v)[4], int keep, bool shifted)
{
    if (shifted) {
        const int sb = 16 - keep, q = sb >> 2, bb = sb & 3;
        uint32_t x[5];
#pragma unroll
        for (int i = 0; i < 5; i++) {
            uint32_t y = 0;
#pragma unroll
            for (int j = 0; j < 4; j++)
                y = (i + j < 4 && q == j) ? v[i + j] : y;
            x[i] = y;
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
            v[i] = __builtin_amdgcn_alignbyte(x[i + 1], x[i], bb);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int kb = keep - 4 * i;
        v[i] = kb >= 4 ? v[i] : (kb <= 0 ? 0u : v[i] & ((1u << (8 * kb)) - 1u));
    }
}

// Each thread moves up to U chunks, `stride` apart (stride = the grid's
// threads), issuing all U loads before it finishes and stores the first.
constexpr int U = 4;

__global__ void __launch_bounds__(256) pack_operands(PackArgs a)
{
    const uint32_t total = a.chunks[0] + a.chunks[1];
    const uint32_t stride = gridDim.x * 256u;
    for (uint32_t c0 = blockIdx.x * 256u + threadIdx.x; c0 < total; c0 += U * stride) {
        uint32_t v[U][4];
        ChunkRef ref[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint32_t c = c0 + u * stride < total ? c0 + u * stride : c0;
            ref[u] = chunk_ref(a, c);
            __builtin_memcpy(v[u], ref[u].src, 16);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (c0 + u * stride < total) {
                if (ref[u].keep < 16)
                    finish_chunk(v[u], ref[u].keep, ref[u].shifted);
                __builtin_memcpy(ref[u].dst, v[u], 16);
            }
        }
    }
}

// Rows shorter than 16 bytes: one chunk per row, read byte by byte.
__global__ void __launch_bounds__(256) pack_short_rows(PackArgs a)
{
    const uint32_t total = a.chunks[0] + a.chunks[1];
    for (uint32_t c = blockIdx.x * 256u + threadIdx.x; c < total; c += gridDim.x * 256u) {
        const int w = c >= a.chunks[0];
        const PackOperand &p = a.op[w];
        const uint32_t q = w ? c - a.chunks[0] : c;
        const uint32_t r = q / a.cpr[w];
        const int64_t b = (int64_t)(q - r * a.cpr[w]) * 16;
        const int64_t left = p.cols * p.es - b;
        const char *src = (const char *)p.src + (int64_t)r * p.ld * p.es + b;
        uint32_t v[4] = {0u, 0u, 0u, 0u};
        char *d = (char *)v;
#pragma unroll
        for (int e = 0; e < 16; e++)
            if (e < left)
                d[e] = src[e];
        __builtin_memcpy((char *)p.dst + (int64_t)q * 16, v, 16);
    }
}

}  // namespace

hipError_t launch_pack(const PackOperand *ops, int n, hipStream_t s)
{
    if (n < 1 || n > 2)
        return hipErrorInvalidValue;
    PackArgs a = {};
    int64_t total = 0;
    bool short_rows = false;
    for (int i = 0; i < n; i++) {
        const PackOperand &p = ops[i];
        if (p.es != 1 && p.es != 2)
            return hipErrorInvalidValue;
        const int64_t cpr = p.cols_p * p.es / 16;
        if (p.rows < 0 || p.cols < 0 || p.cols_p < p.cols || (p.cols_p * p.es) % 16 != 0 ||
            ((uintptr_t)p.dst & 15) != 0 || (p.rows > 0 && cpr == 0))
            return hipErrorInvalidValue;
        const int64_t chunks = p.rows * cpr;
        total += chunks;
        if (total >= (int64_t(1) << 31))
            return hipErrorInvalidValue;
        a.op[i] = p;
        a.chunks[i] = (uint32_t)chunks;
        a.cpr[i] = (uint32_t)(cpr > 0 ? cpr : 1);
        short_rows = short_rows || (chunks > 0 && p.cols * p.es < 16);
    }
    if (total == 0)
        return hipSuccess;
    if (short_rows) {
        const int64_t want = (total + 255) / 256;
        const dim3 grid((unsigned)(want < 4096 ? want : 4096)), block(256);
        hipLaunchKernelGGL(pack_short_rows, grid, block, 0, s, a);
    } else {
        // U chunks per thread; at most 4096 workgroups, the loop strides on
        const int64_t want = (total + 256 * U - 1) / (256 * U);
        const dim3 grid((unsigned)(want < 4096 ? want : 4096)), block(256);
        hipLaunchKernelGGL(pack_operands, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace tg
