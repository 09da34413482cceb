// tg_kernels.h — internal interface between the host dispatcher (tg_api.cpp)
// and the gfx950 kernels (tg_kernels.hip).  Not installed, not part of the ABI.
#ifndef TG_KERNELS_H
#define TG_KERNELS_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tg {

// Kernel arguments.  Sizes are validated by the host to fit 32-bit ints; the
// byte spans a_bytes / b_bytes are the buffer-descriptor ranges of A and B.
struct Params {
    const void *A;   // fp16 or int8 elements (the configuration's element size)
    const void *B;
    const float *bias;
    void *C;
    int M, N, K;
    int lda, ldb, ldc;
    int tiles_m, tiles_n, group_m;
    uint32_t a_bytes, b_bytes;
    int trans_a, trans_b;   // A stored K x M / B stored N x K
    int vec_bias;    // bias allows 16-byte loads
    // K slicing (split-K), used when splits > 1: workgroup row blockIdx.y = z
    // multiplies the K range [z k_split, min((z + 1) k_split, K)) and writes
    // its fp32 (int32 for int8 operands) partial product, without bias, to
    // C + z * c_slice_bytes with leading dimension ldc.
    int splits;
    int k_split;
    int64_t c_slice_bytes;
};

typedef hipError_t (*LaunchFn)(const Params &p, bool f16_out, bool bias, hipStream_t s);

// Sum of the K slices' partial products, in slice order, then bias + ReLU
// and the conversion to C's type.
enum OutKind { kOutF16 = 0, kOutF32 = 1, kOutI32 = 2 };

struct ReduceParams {
    const void *ws;        // splits slices of M x N partials (fp32, or int32 for kOutI32)
    int64_t slice_elems;   // elements between slices
    const float *bias;     // nullptr: plain sum
    void *C;
    int M, N, ldc, splits;
    int vec_ws;            // slices allow 16-byte loads of 4 partials
    int vec_c;             // C rows allow 4-element vector stores
};

hipError_t launch_splitk_reduce(const ReduceParams &r, OutKind out, hipStream_t s);

struct KernelConfig {
    int id;
    int bm, bn, bk, stages, waves_m, waves_n;
    int mfma;         // MFMA block edge: 16 (16x16x32) or 32 (32x32x16)
    int direct;       // 1: direct global->LDS path, 0: register-staged path
    int lds_bytes;
    int ops;          // bit 2*trans_a + trans_b set: that orientation is compiled
    int es;           // operand element size: 2 fp16, 1 int8
    int whole_k;      // 1: serves only K that is a multiple of bk
    const char *name;
};

extern const KernelConfig kConfigs[];
extern const int kNumConfigs;

// The kernels are compiled in up to kMaxShards separate translation units.
constexpr int kMaxShards = 8;

// Launcher of configuration id, or nullptr for an unknown id.
LaunchFn config_launch(int id);

}  // namespace tg

#endif
