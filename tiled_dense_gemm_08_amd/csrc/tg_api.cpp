// tg_api.cpp — host side of libtg.so: argument validation, device checks,
// configuration choice and launch.  See include/tg.h for the contract.
//
// Validation happens before any HIP call, so every argument error is reported
// without touching a device.  The configuration table is static: it was chosen
// offline by an on-device sweep and is only read here (the offline-tune,
// read-only-at-run-time scheme of the lqnn.cn TileLang walkthrough, sections
// 2.3 and 5.3, and the xdnf.cn article, sections 4.3 and 5).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "tg.h"
#include "tg_kernels.h"

namespace {

using tg::kConfigs;
using tg::kNumConfigs;
using tg::KernelConfig;
using tg::Params;

constexpr int64_t kMaxDim = 0x7fffffff;
constexpr int64_t kMaxSpan = int64_t(1) << 31;   // bytes a buffer descriptor may cover

struct Problem {
    const void *A, *B;
    const float *bias;
    void *C;
    int64_t M, N, K, lda, ldb, ldc;
    tg_dtype c_dtype;
    bool fused;
    int op_a, op_b;   // 1: A stored K x M / B stored N x K
};

// Operand element size: int8 operands exactly when C is int32.
int elem_size(const Problem &p) { return p.c_dtype == TG_DTYPE_I32 ? 1 : 2; }

// Largest K for which every int32 partial sum of int8 products is exact:
// |a*b| <= 128*128 = 2^14, and (2^17 - 1) * 2^14 < 2^31.
constexpr int64_t kMaxKInt8 = (int64_t(1) << 17) - 1;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t span_elems(int64_t rows, int64_t cols, int64_t ld)
{
    return (rows == 0 || cols == 0) ? 0 : (rows - 1) * ld + cols;
}

// Stored shape of A and B: rows x cols of the row-major arrays.
int64_t a_rows(const Problem &p) { return p.op_a ? p.K : p.M; }
int64_t a_cols(const Problem &p) { return p.op_a ? p.M : p.K; }
int64_t b_rows(const Problem &p) { return p.op_b ? p.N : p.K; }
int64_t b_cols(const Problem &p) { return p.op_b ? p.K : p.N; }

// Pure argument checks (no HIP calls).
tg_status validate(const Problem &p)
{
    if (p.c_dtype != TG_DTYPE_F16 && p.c_dtype != TG_DTYPE_F32 && p.c_dtype != TG_DTYPE_I32)
        return TG_ERROR_INVALID_VALUE;
    if (p.c_dtype == TG_DTYPE_I32 && p.fused)
        return TG_ERROR_INVALID_VALUE;   // no bias + ReLU epilogue for int32 C
    if ((p.op_a != TG_OP_N && p.op_a != TG_OP_T) || (p.op_b != TG_OP_N && p.op_b != TG_OP_T))
        return TG_ERROR_INVALID_VALUE;
    if (p.M < 0 || p.N < 0 || p.K < 0)
        return TG_ERROR_INVALID_VALUE;
    if (p.lda < a_cols(p) || p.ldb < b_cols(p) || p.ldc < p.N)
        return TG_ERROR_INVALID_VALUE;
    if (p.lda < 0 || p.ldb < 0 || p.ldc < 0)
        return TG_ERROR_INVALID_VALUE;
    if (p.fused && p.bias == nullptr)
        return TG_ERROR_INVALID_VALUE;
    if (p.M == 0 || p.N == 0)
        return TG_SUCCESS;
    if (p.C == nullptr)
        return TG_ERROR_INVALID_VALUE;
    if (p.K > 0 && (p.A == nullptr || p.B == nullptr))
        return TG_ERROR_INVALID_VALUE;
    const uintptr_t c_elem = p.c_dtype == TG_DTYPE_F16 ? 2 : 4;
    const uintptr_t es = elem_size(p);
    if (!aligned(p.A, es) || !aligned(p.B, es) || !aligned(p.C, c_elem) ||
        (p.bias && !aligned(p.bias, 4)))
        return TG_ERROR_INVALID_VALUE;
    if (p.M > kMaxDim || p.N > kMaxDim || p.K > kMaxDim || p.lda > kMaxDim ||
        p.ldb > kMaxDim || p.ldc > kMaxDim)
        return TG_ERROR_UNSUPPORTED;
    if (p.c_dtype == TG_DTYPE_I32 && p.K > kMaxKInt8)
        return TG_ERROR_UNSUPPORTED;
    return TG_SUCCESS;
}

// One operand as the kernels see it: k-major when its stored rows run along M
// or N (A, or B stored N x K), mn-major when they run along K.
struct OperandShape {
    bool kmaj;
    int64_t x;     // M or N
    int64_t ld;
    int tile;      // block_m or block_n
};

bool operand_direct_ok(const OperandShape &o, const Problem &p, int bk)
{
    // every 16-byte chunk entirely inside or entirely outside the operand
    const int64_t es = elem_size(p);
    if ((o.ld * es) % 16 || (o.kmaj ? (p.K * es) % 16 : (o.x * es) % 16))
        return false;
    // lane offsets of rows past the edge (x + tile rows of a k-major operand,
    // block_k + 1 rows of an mn-major one) must stay below 2^32 so that the
    // range check sees them
    if (o.kmaj)
        return es * (o.x + o.tile) * o.ld < (int64_t(1) << 32);
    return es * (bk + 1) * o.ld < kMaxSpan;
}

bool operand_staged_ok(const OperandShape &o, int bk)
{
    return int64_t(o.kmaj ? o.tile : bk) * o.ld < kMaxSpan;   // in-tile offsets fit 31 bits
}

// Whether a configuration can serve this problem (orientation compiled, and
// the alignment and size requirements of its load path).
bool supports(const KernelConfig &c, const Problem &p)
{
    if (!(c.ops & (1 << (2 * p.op_a + p.op_b))) || c.es != elem_size(p))
        return false;
    const OperandShape a{p.op_a == 0, p.M, p.lda, c.bm};
    const OperandShape b{p.op_b == 1, p.N, p.ldb, c.bn};
    if (!c.direct)
        return operand_staged_ok(a, c.bk) && operand_staged_ok(b, c.bk);
    if (!aligned(p.A, 16) || !aligned(p.B, 16))
        return false;
    if (elem_size(p) * span_elems(a_rows(p), a_cols(p), p.lda) >= kMaxSpan ||
        elem_size(p) * span_elems(b_rows(p), b_cols(p), p.ldb) >= kMaxSpan)
        return false;
    return operand_direct_ok(a, p, c.bk) && operand_direct_ok(b, p, c.bk);
}

// ---- configuration table (shape class -> config id), chosen offline ------
#include "tg_dispatch_table.inc"

int choose(const Problem &p)
{
    if (elem_size(p) == 1) {
        const int id = dispatch_int8(p.M, p.N, p.K);
        if (supports(kConfigs[id], p))
            return id;
        return dispatch_int8_fallback(p.M, p.N, p.K);
    }
    const int id = dispatch_table_lookup(p.M, p.N, p.K, p.fused);
    if (id >= 0 && id < kNumConfigs && supports(kConfigs[id], p))
        return id;
    return dispatch_fallback(p.M, p.N, p.K);
}

// ---- device checks (HIP calls) -------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

tg_status check_device(int *dev_out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return TG_ERROR_UNSUPPORTED;
    }
    *dev_out = dev;
    if (dev < 0 || dev >= kMaxDevices)
        return TG_ERROR_UNSUPPORTED;
    int state = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return TG_ERROR_UNSUPPORTED;
        }
        state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(state, std::memory_order_relaxed);
    }
    return state == 1 ? TG_SUCCESS : TG_ERROR_UNSUPPORTED;
}

tg_status check_pointer(const void *ptr, int dev)
{
    if (ptr == nullptr)
        return TG_SUCCESS;
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof(attr));
    if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
        (void)hipGetLastError();   // unregistered host memory: clear the error
        return TG_ERROR_NOT_DEVICE_MEMORY;
    }
    if (attr.type != hipMemoryTypeDevice || attr.device != dev)
        return TG_ERROR_NOT_DEVICE_MEMORY;
    return TG_SUCCESS;
}

tg_status run(int config_id, const Problem &p, hipStream_t stream)
{
    tg_status st = validate(p);
    if (st != TG_SUCCESS)
        return st;
    if (config_id < -1 || config_id >= kNumConfigs)
        return TG_ERROR_INVALID_VALUE;
    if (p.M == 0 || p.N == 0)
        return TG_SUCCESS;
    const int id = config_id >= 0 ? config_id : choose(p);
    const KernelConfig &cfg = kConfigs[id];
    if (!supports(cfg, p))
        return TG_ERROR_UNSUPPORTED;

    int dev = 0;
    if ((st = check_device(&dev)) != TG_SUCCESS)
        return st;
    const bool need_ab = p.K > 0;
    if ((need_ab && ((st = check_pointer(p.A, dev)) != TG_SUCCESS ||
                     (st = check_pointer(p.B, dev)) != TG_SUCCESS)) ||
        (st = check_pointer(p.C, dev)) != TG_SUCCESS ||
        (p.fused && (st = check_pointer(p.bias, dev)) != TG_SUCCESS))
        return st;

    Params k;
    memset(&k, 0, sizeof(k));
    k.A = static_cast<const _Float16 *>(p.A);
    k.B = static_cast<const _Float16 *>(p.B);
    k.bias = p.bias;
    k.C = p.C;
    k.M = (int)p.M;
    k.N = (int)p.N;
    k.K = (int)p.K;
    k.lda = (int)p.lda;
    k.ldb = (int)p.ldb;
    k.ldc = (int)p.ldc;
    k.tiles_m = (int)((p.M + cfg.bm - 1) / cfg.bm);
    k.tiles_n = (int)((p.N + cfg.bn - 1) / cfg.bn);
    k.group_m = 8;
    k.trans_a = p.op_a;
    k.trans_b = p.op_b;
    const int64_t a_span = elem_size(p) * span_elems(a_rows(p), a_cols(p), p.lda);
    const int64_t b_span = elem_size(p) * span_elems(b_rows(p), b_cols(p), p.ldb);
    k.a_bytes = (uint32_t)(a_span < kMaxSpan ? a_span : 0);
    k.b_bytes = (uint32_t)(b_span < kMaxSpan ? b_span : 0);
    const int c_elem = p.c_dtype == TG_DTYPE_F16 ? 2 : 4;
    k.vec_store = (p.ldc % 4 == 0) && aligned(p.C, 4 * c_elem);
    k.line_store = ((p.ldc * c_elem) % 16 == 0) && aligned(p.C, 16);
    k.vec_bias = p.fused && aligned(p.bias, 16);
    if ((int64_t)k.tiles_m * k.tiles_n > kMaxDim)
        return TG_ERROR_UNSUPPORTED;

    (void)hipGetLastError();   // do not report an earlier, unrelated error
    const tg::LaunchFn launch = tg::config_launch(id);
    if (launch == nullptr)
        return TG_ERROR_UNSUPPORTED;
    const hipError_t e = launch(k, p.c_dtype == TG_DTYPE_F16, p.fused, stream);
    return e == hipSuccess ? TG_SUCCESS : TG_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

tg_status tg_gemm(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                  int64_t lda, int64_t ldb, int64_t ldc, tg_dtype c_dtype, hipStream_t stream)
{
    return run(-1, Problem{A, B, nullptr, C, M, N, K, lda, ldb, ldc, c_dtype, false, 0, 0},
               stream);
}

tg_status tg_gemm_bias_relu(const void *A, const void *B, const float *bias, void *C,
                            int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                            int64_t ldc, tg_dtype c_dtype, hipStream_t stream)
{
    if (bias == nullptr)
        return TG_ERROR_INVALID_VALUE;
    return run(-1, Problem{A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, true, 0, 0}, stream);
}

tg_status tg_gemm_ex(tg_op op_a, tg_op op_b, const void *A, const void *B, const float *bias,
                     void *C, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                     int64_t ldc, tg_dtype c_dtype, hipStream_t stream)
{
    return run(-1,
               Problem{A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, bias != nullptr, op_a, op_b},
               stream);
}

tg_status tg_gemm_with_config(int config_id, tg_op op_a, tg_op op_b, const void *A,
                              const void *B, const float *bias, void *C, int64_t M, int64_t N,
                              int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                              tg_dtype c_dtype, hipStream_t stream)
{
    if (config_id < 0 || config_id >= kNumConfigs)
        return TG_ERROR_INVALID_VALUE;
    return run(config_id,
               Problem{A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, bias != nullptr, op_a, op_b},
               stream);
}

const char *tg_status_string(tg_status s)
{
    switch (s) {
    case TG_SUCCESS: return "TG_SUCCESS";
    case TG_ERROR_INVALID_VALUE: return "TG_ERROR_INVALID_VALUE: invalid argument";
    case TG_ERROR_NOT_DEVICE_MEMORY: return "TG_ERROR_NOT_DEVICE_MEMORY: pointer is not device memory of the current device";
    case TG_ERROR_UNSUPPORTED: return "TG_ERROR_UNSUPPORTED: device or problem not supported";
    case TG_ERROR_LAUNCH: return "TG_ERROR_LAUNCH: kernel launch failed";
    }
    return "unknown tg_status";
}

int tg_num_configs(void) { return kNumConfigs; }

tg_status tg_config_info(int id, tg_config_desc *out)
{
    if (id < 0 || id >= kNumConfigs || out == nullptr)
        return TG_ERROR_INVALID_VALUE;
    const KernelConfig &c = kConfigs[id];
    out->id = c.id;
    out->block_m = c.bm;
    out->block_n = c.bn;
    out->block_k = c.bk;
    out->stages = c.stages;
    out->waves_m = c.waves_m;
    out->waves_n = c.waves_n;
    out->mfma = c.mfma;
    out->direct_lds = c.direct;
    out->lds_bytes = c.lds_bytes;
    out->ops = c.ops;
    out->elem_bytes = c.es;
    out->name = c.name;
    return TG_SUCCESS;
}

int tg_config_supports(int id, tg_op op_a, tg_op op_b, const void *A, const void *B,
                       const float *bias, const void *C, int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc, tg_dtype c_dtype)
{
    Problem p{A, B, bias, const_cast<void *>(C), M, N, K, lda, ldb, ldc, c_dtype, bias != nullptr,
              op_a, op_b};
    if (id < 0 || id >= kNumConfigs || validate(p) != TG_SUCCESS)
        return -1;
    return supports(kConfigs[id], p) ? 1 : 0;
}

int tg_select_config(tg_op op_a, tg_op op_b, const void *A, const void *B, const float *bias,
                     const void *C, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                     int64_t ldc, tg_dtype c_dtype)
{
    Problem p{A, B, bias, const_cast<void *>(C), M, N, K, lda, ldb, ldc, c_dtype, bias != nullptr,
              op_a, op_b};
    if (validate(p) != TG_SUCCESS)
        return -1;
    return choose(p);
}

const char *tg_version(void) { return "tg 0.2.0 (gfx950)"; }

}  // extern "C"
