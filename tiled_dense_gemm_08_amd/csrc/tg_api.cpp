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

#include <errno.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <memory>
#include <mutex>
#include <unordered_map>
#include <utility>

#include "tg.h"
#include "tg_diag.h"
#include "tg_attention.h"
#include "tg_ceiling.h"
#include "tg_kernels.h"
#include "tg_pack.h"

namespace {

using tg::kConfigs;
using tg::kNumConfigs;
using tg::KernelConfig;
using tg::Params;

constexpr int64_t kMaxDim = 0x7fffffff;
constexpr int64_t kMaxSpan = int64_t(1) << 31;   // bytes a buffer descriptor may cover
constexpr const char *kTuneMagic = "tg-tuning 1";  // first line of a tuning cache file

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

// Every 16-byte chunk of the operand's rows lies entirely inside or entirely
// outside the operand (given a 16-byte-aligned base).
bool chunks_aligned(const OperandShape &o, const Problem &p)
{
    const int64_t es = elem_size(p);
    return (o.ld * es) % 16 == 0 && (o.kmaj ? (p.K * es) % 16 : (o.x * es) % 16) == 0;
}

bool operand_direct_ok(const OperandShape &o, const Problem &p, int bk)
{
    if (!chunks_aligned(o, p))
        return false;
    const int64_t es = elem_size(p);
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
    if (c.whole_k && p.K % c.bk != 0)
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

// ---- dispatch ---------------------------------------------------------------
// A problem is served, in this order, by: the run-time tuning cache (exact
// shape records written by the sweep and loaded with tg_tuning_load or
// TG_TUNING_FILE), the compiled exact-shape table, the least predicted time of
// the compiled cost model (fitted offline to on-device timings on a grid of
// shapes), and finally the register-staged fallback, which runs any alignment.
// Each step is taken only if its configuration can run the problem.
#include "tg_dispatch_table.inc"
#include "tg_cost_model.inc"

constexpr int kModelCUs = 256;   // compute units of an MI355X

// Fitted time at K: piecewise linear through the grid values, the end
// stretches extended, and never below a tenth of the smallest grid value.
double model_interp(const int64_t *k, const double *v, int64_t K)
{
    int i = 0;
    while (i + 2 < kModelNK && K > k[i + 1])
        i++;
    const double t = v[i] + (v[i + 1] - v[i]) * (double)(K - k[i]) / (double)(k[i + 1] - k[i]);
    double lo = v[0];
    for (int j = 1; j < kModelNK; j++)
        lo = v[j] < lo ? v[j] : lo;
    return t > 0.1 * lo ? t : 0.1 * lo;
}

// Predicted time of configuration c: tiles = ceil(M/BM) * ceil(N/BN)
// workgroups take R = tiles / slots rounds on the chip's CUs; each full round
// costs t_full(K), and a partial round filling a fraction f of the slots
// costs t_min(K) + f * (t_full(K) - t_min(K)).
double model_rounds_time(const ModelRow &r, double workgroups, int64_t K)
{
    const double R = workgroups / (double)(kModelCUs * r.per_cu);
    const double fl = floor(R), f = R - fl;
    double a = fl, b = 0.0;
    if (f > 1e-12) {
        a = fl + f;
        b = 1.0 - f;
    }
    return a * model_interp(r.k, r.t_full, K) + b * model_interp(r.k, r.t_min, K);
}

double n_tiles(const KernelConfig &c, const Problem &p)
{
    return (double)((p.M + c.bm - 1) / c.bm) * (double)((p.N + c.bn - 1) / c.bn);
}

double model_time(const ModelRow &r, const KernelConfig &c, const Problem &p)
{
    return model_rounds_time(r, n_tiles(c, p), p.K);
}

// Whether the operands have the 16-byte layout the direct loads need; the
// register-staged kernels run at a different speed on such operands, and the
// model has a row for each case.
bool operands_aligned(const Problem &p)
{
    return aligned(p.A, 16) && aligned(p.B, 16) &&
           chunks_aligned(OperandShape{p.op_a == 0, p.M, p.lda, 0}, p) &&
           chunks_aligned(OperandShape{p.op_b == 1, p.N, p.ldb, 0}, p);
}

bool has_model_row(int id, int padded)
{
    for (const ModelRow &r : kModel)
        if (r.id == id && r.padded == padded)
            return true;
    return false;
}

// The model row to use for configuration `r.id` on this problem: its row for
// the problem's operand layout, or its only row.
bool row_applies(const ModelRow &r, const Problem &p, int pad)
{
    if (r.id < 0 || r.id >= kNumConfigs || !supports(kConfigs[r.id], p))
        return false;
    return r.padded == pad || !has_model_row(r.id, pad);
}

// The modelled configuration with the least predicted time that can run the
// problem (ties: the lower id), or -1; its predicted time in *t_out.
// direct_only: among the direct-copy configurations only.
int model_lookup(const Problem &p, double *t_out = nullptr, bool direct_only = false)
{
    const int pad = operands_aligned(p) ? 0 : 1;
    int best = -1;
    double best_t = 0.0;
    for (const ModelRow &r : kModel) {
        if (!row_applies(r, p, pad) || (direct_only && !kConfigs[r.id].direct))
            continue;
        const double t = model_time(r, kConfigs[r.id], p);
        if (best < 0 || t < best_t || (t == best_t && r.id < best)) {
            best = r.id;
            best_t = t;
        }
    }
    if (t_out)
        *t_out = best_t;
    return best;
}

// ---- run-time tuning cache ----------------------------------------------------
// Exact-shape records, read-only once loaded: a load builds a new table and
// swaps it in whole, so concurrent calls see either the old or the new one.
struct TuneKey {
    int64_t M, N, K;
    int op_a, op_b, c_dtype, fused;
    bool operator==(const TuneKey &o) const
    {
        return M == o.M && N == o.N && K == o.K && op_a == o.op_a && op_b == o.op_b &&
               c_dtype == o.c_dtype && fused == o.fused;
    }
};

struct TuneKeyHash {
    size_t operator()(const TuneKey &k) const
    {
        uint64_t h = 0x9e3779b97f4a7c15ull;
        for (uint64_t v : {(uint64_t)k.M, (uint64_t)k.N, (uint64_t)k.K,
                           (uint64_t)(k.op_a | k.op_b << 1 | k.fused << 2 | k.c_dtype << 3)}) {
            h ^= v + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
        }
        return (size_t)h;
    }
};

using TuneTable = std::unordered_map<TuneKey, int, TuneKeyHash>;

constexpr int kMaxTuneRecords = 1 << 20;
constexpr size_t kMaxTuneLine = 1024;

std::mutex g_tune_mu;
std::shared_ptr<const TuneTable> g_tune;   // guarded by g_tune_mu; null = empty
std::atomic<bool> g_tune_any{false};
std::atomic<uint64_t> g_tune_gen{0};       // bumped by every change of the table
std::once_flag g_tune_env_once;

TuneKey tune_key(const Problem &p)
{
    return TuneKey{p.M, p.N, p.K, p.op_a, p.op_b, (int)p.c_dtype, p.fused ? 1 : 0};
}

bool parse_int(const char *s, int64_t lo, int64_t hi, int64_t *out)
{
    char *end = nullptr;
    errno = 0;
    const long long v = strtoll(s, &end, 10);
    if (errno || end == s || *end != '\0' || v < lo || v > hi)
        return false;
    *out = v;
    return true;
}

// One record line: M N K op_a op_b c_dtype fused config name tflops.
// Returns 1 for a record, 0 for a stale record (the configuration id names
// another kernel in this build, or one that cannot serve the record's
// orientation or element type), -1 for a malformed line.
int parse_record(char *line, TuneKey *key, int *id)
{
    char *tok[11];
    int n = 0;
    for (char *save = nullptr, *t = strtok_r(line, " \t", &save); t != nullptr;
         t = strtok_r(nullptr, " \t", &save)) {
        if (n == 11)
            return -1;
        tok[n++] = t;
    }
    if (n != 10)
        return -1;
    int64_t M, N, K, fused, cid;
    if (!parse_int(tok[0], 0, kMaxDim, &M) || !parse_int(tok[1], 0, kMaxDim, &N) ||
        !parse_int(tok[2], 0, kMaxDim, &K) || !parse_int(tok[6], 0, 1, &fused) ||
        !parse_int(tok[7], 0, kMaxDim, &cid))
        return -1;
    int ops[2];
    for (int i = 0; i < 2; i++) {
        if (strcmp(tok[3 + i], "N") == 0)
            ops[i] = TG_OP_N;
        else if (strcmp(tok[3 + i], "T") == 0)
            ops[i] = TG_OP_T;
        else
            return -1;
    }
    tg_dtype dt;
    if (strcmp(tok[5], "f16") == 0)
        dt = TG_DTYPE_F16;
    else if (strcmp(tok[5], "f32") == 0)
        dt = TG_DTYPE_F32;
    else if (strcmp(tok[5], "i32") == 0)
        dt = TG_DTYPE_I32;
    else
        return -1;
    if (dt == TG_DTYPE_I32 && fused)
        return -1;
    char *end = nullptr;
    const double tflops = strtod(tok[9], &end);
    if (end == tok[9] || *end != '\0' || !(tflops >= 0.0) || tflops > 1e9)
        return -1;
    *key = TuneKey{M, N, K, ops[0], ops[1], (int)dt, (int)fused};
    *id = (int)cid;
    if (cid >= kNumConfigs)
        return 0;
    const KernelConfig &c = kConfigs[cid];
    const int es = dt == TG_DTYPE_I32 ? 1 : 2;
    if (strcmp(c.name, tok[8]) != 0 || !(c.ops & (1 << (2 * ops[0] + ops[1]))) || c.es != es)
        return 0;
    return 1;
}

void strip_eol(char *s)
{
    size_t n = strlen(s);
    while (n > 0 && (s[n - 1] == '\n' || s[n - 1] == '\r' || s[n - 1] == ' ' || s[n - 1] == '\t'))
        s[--n] = '\0';
}

tg_status read_tuning_file(const char *path, TuneTable *table, int *loaded, int *skipped,
                           int *error_line)
{
    if (loaded)
        *loaded = 0;
    if (skipped)
        *skipped = 0;
    if (error_line)
        *error_line = 0;
    FILE *f = fopen(path, "r");
    if (f == nullptr)
        return TG_ERROR_FILE;
    char buf[kMaxTuneLine + 2];
    int line_no = 0, n_ok = 0, n_stale = 0;
    tg_status st = TG_SUCCESS;
    while (fgets(buf, sizeof(buf), f) != nullptr) {
        line_no++;
        if (strlen(buf) > kMaxTuneLine) {   // line longer than any record
            st = TG_ERROR_INVALID_VALUE;
            break;
        }
        strip_eol(buf);
        if (line_no == 1) {
            if (strcmp(buf, kTuneMagic) != 0) {
                st = TG_ERROR_INVALID_VALUE;
                break;
            }
            continue;
        }
        const char *q = buf;
        while (*q == ' ' || *q == '\t')
            q++;
        if (*q == '\0' || *q == '#')
            continue;
        TuneKey key;
        int id = -1;
        const int r = parse_record(buf, &key, &id);
        if (r < 0 || n_ok + n_stale >= kMaxTuneRecords) {
            st = TG_ERROR_INVALID_VALUE;
            break;
        }
        if (r == 0) {
            n_stale++;
            continue;
        }
        (*table)[key] = id;   // a later record for the same key wins
        n_ok++;   // counts toward the record limit
    }
    if (st == TG_SUCCESS && ferror(f))
        st = TG_ERROR_FILE;
    if (st == TG_SUCCESS && line_no == 0)
        st = TG_ERROR_INVALID_VALUE;   // empty file: no magic line
    fclose(f);
    if (error_line)
        *error_line = st == TG_ERROR_INVALID_VALUE ? (line_no == 0 ? 1 : line_no) : 0;
    if (st == TG_SUCCESS && loaded)
        *loaded = (int)table->size();
    if (st == TG_SUCCESS && skipped)
        *skipped = n_stale;
    return st;
}

void publish(std::shared_ptr<const TuneTable> t)
{
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_tune = std::move(t);
    g_tune_any.store(g_tune != nullptr && !g_tune->empty(), std::memory_order_release);
    g_tune_gen.fetch_add(1, std::memory_order_acq_rel);
}

// TG_TUNING_FILE: loaded once, before the first call that reads or changes
// the cache.  A file that does not load leaves the cache empty and is
// reported once on stderr (a GEMM call has no status for it).
void load_env_cache()
{
    const char *path = getenv("TG_TUNING_FILE");
    if (path == nullptr || *path == '\0')
        return;
    auto t = std::make_shared<TuneTable>();
    int line = 0;
    const tg_status st = read_tuning_file(path, t.get(), nullptr, nullptr, &line);
    if (st != TG_SUCCESS) {
        fprintf(stderr, "libtg: TG_TUNING_FILE=%s not loaded (%s, line %d)\n", path,
                tg_status_string(st), line);
        return;
    }
    publish(std::move(t));
}

void ensure_env_cache() { std::call_once(g_tune_env_once, load_env_cache); }

int tuned_lookup(const Problem &p)
{
    ensure_env_cache();
    if (!g_tune_any.load(std::memory_order_acquire))
        return -1;
    std::shared_ptr<const TuneTable> t;
    {
        std::lock_guard<std::mutex> lk(g_tune_mu);
        t = g_tune;
    }
    if (!t)
        return -1;
    const auto it = t->find(tune_key(p));
    return it == t->end() ? -1 : it->second;
}

int choose(const Problem &p)
{
    const int tuned = tuned_lookup(p);
    if (tuned >= 0 && supports(kConfigs[tuned], p))
        return tuned;
    const int exact = dispatch_exact(p.M, p.N, p.K, p.fused, elem_size(p));
    if (exact >= 0 && supports(kConfigs[exact], p))
        return exact;
    const int modelled = model_lookup(p);
    if (modelled >= 0)
        return modelled;
    return elem_size(p) == 1 ? dispatch_int8_fallback(p.M, p.N, p.K)
                             : dispatch_fallback(p.M, p.N, p.K);
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

// ptr is device memory of device dev and [ptr, ptr + bytes) lies inside the
// allocation that holds it (hipMemGetAddressRange: the whole hipMalloc block,
// so a framework's sub-allocation is checked against its pool block).
// TG_ERROR_INVALID_VALUE when the span runs past the allocation's end.
tg_status check_span(const void *ptr, uint64_t bytes, int dev)
{
    if (ptr == nullptr || bytes == 0)
        return TG_SUCCESS;
    tg_status st = check_pointer(ptr, dev);
    if (st != TG_SUCCESS)
        return st;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)ptr) != hipSuccess) {
        (void)hipGetLastError();
        return TG_ERROR_NOT_DEVICE_MEMORY;
    }
    const uintptr_t lo = (uintptr_t)base, at = (uintptr_t)ptr;
    if (at < lo || at - lo > size || (uint64_t)(size - (at - lo)) < bytes)
        return TG_ERROR_INVALID_VALUE;
    return TG_SUCCESS;
}

// Kernel arguments of configuration cfg for problem p (no K slicing).
tg_status make_params(const KernelConfig &cfg, const Problem &p, Params *out)
{
    Params &k = *out;
    memset(&k, 0, sizeof(k));
    k.A = p.A;
    k.B = p.B;
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
    k.vec_bias = p.fused && aligned(p.bias, 16);
    k.splits = 1;
    if ((int64_t)k.tiles_m * k.tiles_n > kMaxDim)
        return TG_ERROR_UNSUPPORTED;
    return TG_SUCCESS;
}

// The problem's buffers are device memory of the current device and every
// element the call reads or writes lies inside its allocation: A and B over
// their stored rows (when K > 0), C over its M rows and bias over N floats.
tg_status check_problem_pointers(const Problem &p, int *dev)
{
    tg_status st;
    if ((st = check_device(dev)) != TG_SUCCESS)
        return st;
    const uint64_t es = elem_size(p), ce = p.c_dtype == TG_DTYPE_F16 ? 2 : 4;
    if (p.K > 0 &&
        ((st = check_span(p.A, es * span_elems(a_rows(p), a_cols(p), p.lda), *dev)) != TG_SUCCESS ||
         (st = check_span(p.B, es * span_elems(b_rows(p), b_cols(p), p.ldb), *dev)) != TG_SUCCESS))
        return st;
    if ((st = check_span(p.C, ce * span_elems(p.M, p.N, p.ldc), *dev)) != TG_SUCCESS)
        return st;
    if (p.fused && (st = check_span(p.bias, 4 * (uint64_t)p.N, *dev)) != TG_SUCCESS)
        return st;
    return TG_SUCCESS;
}

tg_status launch_config(int id, const Params &k, bool f16_out, bool bias, hipStream_t stream)
{
    (void)hipGetLastError();   // do not report an earlier, unrelated error
    const tg::LaunchFn launch = tg::config_launch(id);
    if (launch == nullptr)
        return TG_ERROR_UNSUPPORTED;
    return launch(k, f16_out, bias, stream) == hipSuccess ? TG_SUCCESS : TG_ERROR_LAUNCH;
}

// ---- split-K ------------------------------------------------------------------
// K is cut into slices of k_split elements (a multiple of the configuration's
// K step); every slice's product runs as its own row of workgroups and
// writes an fp32 (int32) partial product to the caller's workspace; a second
// kernel sums the partials in slice order, adds the bias, applies ReLU and
// converts.  The order is fixed, so results are reproducible run to run.
constexpr int kMaxSplits = 64;
constexpr int kSplitCandidates[] = {2, 3, 4, 6, 8, 12, 16, 24, 32};
// Cost of slicing on top of the sliced GEMM's modelled rounds: a fixed part
// (the second launch), the bytes the reduction moves at an effective rate,
// and a per-slice part (each slice's prologue and partial write).  Fitted to
// on-device timings of every kernel at 2..32 slices on shapes with
// M, N in 128..2048 and K in 2048..32768 (microseconds, bytes/us).
constexpr double kReduceFixedUs = 4.5;
constexpr double kReduceBytesPerUs = 4.5e6;
constexpr double kSliceUs = 0.3;

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int64_t slice_k(int64_t K, int splits, int bk)
{
    const int64_t per = (K + splits - 1) / splits;
    return (per + bk - 1) / bk * bk;
}

int64_t slice_count(int64_t K, int64_t k_split) { return k_split > 0 ? (K + k_split - 1) / k_split : 1; }

// Workspace bytes of the slices' partial products (fp32 or int32, M x N each).
int64_t partial_bytes(const Problem &p, int64_t slices) { return slices * p.M * p.N * 4; }

double reduce_time(const Problem &p, int64_t slices)
{
    const double c_bytes = p.c_dtype == TG_DTYPE_F16 ? 2.0 : 4.0;
    const double bytes = (double)slices * (double)p.M * (double)p.N * 4.0 +
                         (double)p.M * (double)p.N * c_bytes;
    return kReduceFixedUs + bytes / kReduceBytesPerUs + kSliceUs * (double)slices;
}

// Configurations that the chooser runs unsliced only, unless the caller names
// both the configuration and a slice count: the 4-stage 64x64 kernel's model
// row is fitted on unsliced launches, and on the slicing calibration shapes
// its sliced predictions chose kernels 1.056x slower than the fastest on
// average (up to 1.27x), against 1.015x without them.
constexpr int kNoAutoSlicing[] = {21};

bool auto_slicing_ok(int id)
{
    for (int x : kNoAutoSlicing)
        if (x == id)
            return false;
    return true;
}

struct SplitChoice {
    int id;
    int64_t slices;    // 1: no K slicing
    int64_t k_split;   // K elements per slice
    double t;
};

// Least predicted time over the modelled configurations that can run the
// problem and the slice counts whose partials fit in ws_bytes; `only_id` /
// `only_splits` restrict the search (-1 / 0: free), `direct_only` keeps the
// direct-copy configurations only.  Returns id -1 when no modelled
// configuration applies.
SplitChoice choose_split(const Problem &p, size_t ws_bytes, int only_id, int only_splits,
                         bool direct_only = false)
{
    const int pad = operands_aligned(p) ? 0 : 1;
    SplitChoice best{-1, 1, p.K, 0.0};
    for (const ModelRow &r : kModel) {
        if ((only_id >= 0 && r.id != only_id) || !row_applies(r, p, pad) ||
            (direct_only && !kConfigs[r.id].direct))
            continue;
        const KernelConfig &c = kConfigs[r.id];
        auto consider = [&](int64_t slices, int64_t kk) {
            const double t = slices > 1
                                 ? model_rounds_time(r, n_tiles(c, p) * (double)slices, kk) +
                                       reduce_time(p, slices)
                                 : model_time(r, c, p);
            if (best.id < 0 || t < best.t ||
                (t == best.t && (slices < best.slices || (slices == best.slices && r.id < best.id))))
                best = SplitChoice{r.id, slices, kk, t};
        };
        if (only_splits <= 1)
            consider(1, p.K);
        if (only_splits == 1 || (only_splits == 0 && !auto_slicing_ok(r.id)))
            continue;
        const int one[] = {only_splits};
        const int *cand = only_splits > 1 ? one : kSplitCandidates;
        const int ncand = only_splits > 1 ? 1 : (int)(sizeof(kSplitCandidates) / sizeof(int));
        for (int i = 0; i < ncand; i++) {
            const int64_t kk = slice_k(p.K, cand[i], c.bk);
            const int64_t slices = slice_count(p.K, kk);
            if (slices <= 1 || (uint64_t)partial_bytes(p, slices) > (uint64_t)ws_bytes)
                continue;
            consider(slices, kk);
        }
    }
    return best;
}

// ---- packed operands -----------------------------------------------------------
// An operand the direct global->LDS copies cannot take (base not 16-byte
// aligned, or leading dimension or row length not a multiple of 16 bytes) is
// otherwise served by the register-staged kernels, which hide less memory
// latency.  With a workspace the dispatcher may instead copy it there first,
// in a packed layout: the same stored rows, each padded with zeros to a
// multiple of 16 bytes, which is also the copy's leading dimension
// (tg_pack.hip).  The direct kernel then runs on the copy; the kernel's K is K
// rounded up to a whole 16-byte chunk (the padding holds zeros, and the rows
// past K of an operand whose rows run along K lie past its copy range, which
// reads zeros).  Copy time: a fixed part (the extra launch) and the bytes read
// and written at an effective rate; fitted to on-device traces of the copy
// kernel for copies of 0.5 MB .. 0.5 GB (3.4 us + bytes / 6.1e6 per us),
// rounded up.
constexpr double kPackFixedUs = 4.0;
constexpr double kPackBytesPerUs = 5.5e6;

bool operand_direct_layout(const Problem &p, bool is_a)
{
    const void *ptr = is_a ? p.A : p.B;
    const OperandShape o = is_a ? OperandShape{p.op_a == 0, p.M, p.lda, 0}
                                : OperandShape{p.op_b == 1, p.N, p.ldb, 0};
    return aligned(ptr, 16) && chunks_aligned(o, p);
}

// What one call runs: configuration `id` on the problem `kp` (p itself, or p
// with packed copies of some operands), unsliced or in `slices` K slices.
// Workspace layout: the packed copies first (each rounded up to 256 bytes),
// then the slices' partial products.
struct Plan {
    int id = -1;
    int64_t slices = 1, k_split = 0;
    bool pack[2] = {false, false};
    tg::PackOperand op[2] = {};        // the copies (src set, dst set at run time)
    int64_t copy_bytes[2] = {0, 0};
    int64_t range[2] = {0, 0};         // buffer ranges of the kernel's operands when packing
    Problem kp{};                      // the problem the kernel sees (copy pointers at run time)
    size_t pack_bytes = 0;             // workspace of the copies
    size_t part_bytes = 0;             // workspace of the partial products
    double t = 0.0;                    // modelled time (0 when not modelled)
    size_t ws_used() const { return pack_bytes + part_bytes; }
};

// Packed geometry of p: which operands are copied, the copies' sizes and the
// problem the direct kernel sees (`chk`: the same with stand-in 16-byte
// aligned addresses for the eligibility checks).  False when a copy would
// span 2 GiB or more, or the copies still do not suit the direct kernels.
bool pack_geometry(const Problem &p, Plan *pl, Problem *chk)
{
    const int64_t es = elem_size(p), ce = 16 / es;
    pl->pack[0] = !operand_direct_layout(p, true);
    pl->pack[1] = !operand_direct_layout(p, false);
    Problem kp = p;
    kp.K = round_up(p.K, ce);
    *chk = kp;
    for (int w = 0; w < 2; w++) {
        const bool is_a = w == 0;
        const bool kmaj = is_a ? p.op_a == 0 : p.op_b == 1;
        const int64_t rows = is_a ? a_rows(p) : b_rows(p);
        const int64_t cols = is_a ? a_cols(p) : b_cols(p);
        const int64_t ld = is_a ? p.lda : p.ldb;
        if (!pl->pack[w]) {
            // unpacked: its own rows; an operand whose rows run along K keeps
            // its K rows in range, so the kernel's extra K rows read zeros
            pl->range[w] = es * span_elems(rows, cols, ld);
            continue;
        }
        const int64_t cols_p = round_up(cols, ce);
        const int64_t copy = rows * cols_p * es;
        if (copy >= kMaxSpan)
            return false;
        pl->op[w] = tg::PackOperand{is_a ? p.A : p.B, nullptr, rows, cols, ld, cols_p, (int)es};
        pl->copy_bytes[w] = copy;
        pl->range[w] = copy;
        pl->pack_bytes += (size_t)round_up(copy, 256);
        if (is_a) {
            kp.lda = cols_p;
            chk->lda = cols_p;
            if (!kmaj)
                chk->M = cols_p;
        } else {
            kp.ldb = cols_p;
            chk->ldb = cols_p;
            if (!kmaj)
                chk->N = cols_p;
        }
    }
    chk->A = pl->pack[0] ? reinterpret_cast<const void *>(uintptr_t(256)) : p.A;
    chk->B = pl->pack[1] ? reinterpret_cast<const void *>(uintptr_t(512)) : p.B;
    chk->K = kp.K;
    pl->kp = kp;
    return operands_aligned(*chk);
}

double pack_time(const Plan &pl, const Problem &p)
{
    const int64_t es = elem_size(p);
    double bytes = 0.0;
    for (int w = 0; w < 2; w++)
        if (pl.pack[w])
            bytes += (double)(es * span_elems(w ? b_rows(p) : a_rows(p), w ? b_cols(p) : a_cols(p),
                                              w ? p.ldb : p.lda) +
                              pl.copy_bytes[w]);
    return kPackFixedUs + bytes / kPackBytesPerUs;
}

// The slice count of a plan on problem q (the operands as passed, or their
// packed copies) for configuration id (-1: the dispatcher's) with ws_bytes of
// workspace left: splits 0 = the modelled choice among 1 and the slice counts
// whose partials fit; 1 = unsliced; n > 1 = n slices.
void plan_slices(Plan *pl, const Problem &q, int id, int splits, size_t ws_bytes)
{
    pl->slices = 1;
    pl->k_split = q.K;
    if (splits == 0 && q.K > 0 && ws_bytes > 0) {
        // exact records of the tuning cache and compiled table still decide
        // an unsliced call of the dispatcher
        const SplitChoice sc = choose_split(q, ws_bytes, id, 0);
        if (sc.id >= 0) {
            pl->id = sc.id;
            pl->slices = sc.slices;
            pl->k_split = sc.k_split;
            pl->t = sc.t;
        }
        if (pl->slices <= 1)
            pl->id = id >= 0 ? id : choose(q);
    } else if (splits > 1 && q.K > 0) {
        if (id < 0) {
            const SplitChoice sc = choose_split(q, SIZE_MAX, -1, splits);
            id = sc.id >= 0 ? sc.id : choose(q);
        }
        pl->id = id;
        pl->k_split = slice_k(q.K, splits, kConfigs[id].bk);
        pl->slices = slice_count(q.K, pl->k_split);
    } else {
        pl->id = id >= 0 ? id : choose(q);
    }
    pl->part_bytes = pl->slices > 1 ? (size_t)partial_bytes(q, pl->slices) : 0;
}

// The plan of a call without workspace, or of one that names its
// configuration or slice count (config_id -1: the dispatcher's
// configuration).  No copies, except that a named direct configuration that
// cannot take an operand as passed runs on packed copies of the operands
// that need it, when ws_bytes holds them.
tg_status plan_fixed(const Problem &p, int config_id, int splits, size_t ws_bytes, Plan *out)
{
    Plan pl;
    pl.kp = p;
    if (config_id >= 0 && !supports(kConfigs[config_id], p)) {
        Problem chk;
        if (!kConfigs[config_id].direct || ws_bytes == 0 || !pack_geometry(p, &pl, &chk) ||
            !supports(kConfigs[config_id], chk))
            return TG_ERROR_UNSUPPORTED;
        if (pl.pack_bytes > ws_bytes)
            return TG_ERROR_WORKSPACE;
        plan_slices(&pl, chk, config_id, splits, ws_bytes - pl.pack_bytes);
        // partials of the real output (chk's M or N may be rounded up to the
        // copy's row length, so the fit was checked conservatively)
        pl.part_bytes = pl.slices > 1 ? (size_t)partial_bytes(p, pl.slices) : 0;
        *out = pl;
        return TG_SUCCESS;
    }
    plan_slices(&pl, p, config_id, splits, ws_bytes);
    *out = pl;
    return TG_SUCCESS;
}

// The dispatcher's plan with a workspace of ws_bytes: the fastest modelled of
// (a) the operands as passed, unsliced or in K slices whose partials fit, and
// (b) packed copies of the operands that rule out the direct copies, then a
// direct configuration on them, unsliced or sliced, copies and partials
// together within ws_bytes.  A tuning-cache record for the exact problem is
// run as recorded (unpacked, unsliced).
Plan plan_auto(const Problem &p, size_t ws_bytes)
{
    Plan base;
    const int tuned = tuned_lookup(p);
    if (tuned >= 0 && supports(kConfigs[tuned], p)) {
        base.id = tuned;
        base.kp = p;
        base.k_split = p.K;
        return base;
    }
    plan_fixed(p, -1, 0, ws_bytes, &base);
    if (p.K == 0 || operands_aligned(p))
        return base;
    double t_base = base.t;
    if (base.t == 0.0 && model_lookup(p, &t_base) < 0)
        return base;   // nothing modelled to compare with
    Plan pk;
    Problem chk;
    if (!pack_geometry(p, &pk, &chk) || pk.pack_bytes > ws_bytes)
        return base;
    const SplitChoice sc = choose_split(chk, ws_bytes - pk.pack_bytes, -1, 0, true);
    if (sc.id < 0)
        return base;
    pk.id = sc.id;
    pk.slices = sc.slices;
    pk.k_split = sc.k_split;
    if (sc.slices <= 1) {
        // a measured exact-shape record for the copies' problem overrides the
        // model's kernel (the predicted time still decides whether to pack)
        const int exact = dispatch_exact(chk.M, chk.N, chk.K, chk.fused, elem_size(chk));
        if (exact >= 0 && kConfigs[exact].direct && supports(kConfigs[exact], chk))
            pk.id = exact;
    } else {
        pk.part_bytes = (size_t)partial_bytes(p, sc.slices);
    }
    pk.t = sc.t + pack_time(pk, p);
    return pk.t < t_base ? pk : base;
}

// ---- launches -------------------------------------------------------------------
// Runs the plan: the copies into the workspace, then the kernel on the
// problem it sees -- into C, or into the workspace's partial products
// followed by their reduction into C.  The workspace has been checked.
tg_status execute(const Plan &pl, const Problem &p, char *ws, hipStream_t stream)
{
    Problem kp = pl.kp;
    const bool packed = pl.pack[0] || pl.pack[1];
    if (packed) {
        tg::PackOperand ops[2];
        int n = 0;
        size_t at = 0;
        for (int w = 0; w < 2; w++) {
            if (!pl.pack[w])
                continue;
            ops[n] = pl.op[w];
            ops[n].dst = ws + at;
            (w == 0 ? kp.A : kp.B) = ws + at;
            at += (size_t)round_up(pl.copy_bytes[w], 256);
            n++;
        }
        (void)hipGetLastError();
        if (tg::launch_pack(ops, n, stream) != hipSuccess)
            return TG_ERROR_LAUNCH;
    }
    const KernelConfig &cfg = kConfigs[pl.id];
    tg_status st;
    if (pl.slices <= 1) {
        Params k;
        if ((st = make_params(cfg, kp, &k)) != TG_SUCCESS)
            return st;
        if (packed) {
            k.a_bytes = (uint32_t)pl.range[0];
            k.b_bytes = (uint32_t)pl.range[1];
        }
        return launch_config(pl.id, k, kp.c_dtype == TG_DTYPE_F16, kp.fused, stream);
    }
    // the slices' partial products: M x N, leading dimension N, fp32 (int32)
    Problem part = kp;
    part.C = ws + pl.pack_bytes;
    part.ldc = p.N;
    part.bias = nullptr;
    part.fused = false;
    part.c_dtype = elem_size(p) == 1 ? TG_DTYPE_I32 : TG_DTYPE_F32;
    Params k;
    if ((st = make_params(cfg, part, &k)) != TG_SUCCESS)
        return st;
    if (packed) {
        k.a_bytes = (uint32_t)pl.range[0];
        k.b_bytes = (uint32_t)pl.range[1];
    }
    k.splits = (int)pl.slices;
    k.k_split = (int)pl.k_split;
    k.c_slice_bytes = p.M * p.N * 4;
    if ((st = launch_config(pl.id, k, false, false, stream)) != TG_SUCCESS)
        return st;
    tg::ReduceParams r;
    r.ws = part.C;
    r.slice_elems = p.M * p.N;
    r.bias = p.fused ? p.bias : nullptr;
    r.C = p.C;
    r.M = (int)p.M;
    r.N = (int)p.N;
    r.ldc = (int)p.ldc;
    r.splits = (int)pl.slices;
    r.vec_ws = p.N % 4 == 0;
    const int c_elem = p.c_dtype == TG_DTYPE_F16 ? 2 : 4;
    r.vec_c = p.ldc % 4 == 0 && aligned(p.C, 4 * c_elem);
    const tg::OutKind kind = p.c_dtype == TG_DTYPE_F16   ? tg::kOutF16
                             : p.c_dtype == TG_DTYPE_F32 ? tg::kOutF32
                                                         : tg::kOutI32;
    return tg::launch_splitk_reduce(r, kind, stream) == hipSuccess ? TG_SUCCESS : TG_ERROR_LAUNCH;
}

// ---- plan cache -----------------------------------------------------------------
// Choosing a plan walks the cost model's rows and slice counts (a few
// microseconds, as long as a small GEMM takes on the device).  A plan is a
// function of the problem's sizes, leading dimensions, orientation, output
// type, epilogue, the low four bits of the A and B addresses (which decide
// the load path), the named configuration and slice count, the workspace
// size and the tuning cache's contents; each host thread keeps its last few
// plans under that key and rebinds the buffer pointers on a hit.
struct PlanKey {
    int64_t M, N, K, lda, ldb, ldc;
    int op_a, op_b, c_dtype, fused, config_id, splits;
    uint32_t align;
    uint64_t ws_bytes, tune_gen;
    bool operator==(const PlanKey &o) const
    {
        return M == o.M && N == o.N && K == o.K && lda == o.lda && ldb == o.ldb &&
               ldc == o.ldc && op_a == o.op_a && op_b == o.op_b && c_dtype == o.c_dtype &&
               fused == o.fused && config_id == o.config_id && splits == o.splits &&
               align == o.align && ws_bytes == o.ws_bytes && tune_gen == o.tune_gen;
    }
};

struct PlanSlot {
    bool used = false;
    PlanKey key{};
    Plan plan;
};

constexpr int kPlanSlots = 8;
thread_local PlanSlot t_plans[kPlanSlots];
thread_local int t_plan_next = 0;

PlanKey plan_key(const Problem &p, int config_id, int splits, size_t ws_bytes)
{
    ensure_env_cache();
    const uint32_t align = (uint32_t)((reinterpret_cast<uintptr_t>(p.A) & 15) |
                                      ((reinterpret_cast<uintptr_t>(p.B) & 15) << 4));
    return PlanKey{p.M, p.N, p.K, p.lda, p.ldb, p.ldc, p.op_a, p.op_b, (int)p.c_dtype,
                   p.fused ? 1 : 0, config_id, splits, align, (uint64_t)ws_bytes,
                   g_tune_gen.load(std::memory_order_acquire)};
}

// A cached plan for p, with p's pointers bound in, or false.
bool plan_cached(const PlanKey &k, const Problem &p, Plan *out)
{
    for (const PlanSlot &sl : t_plans) {
        if (sl.used && sl.key == k) {
            *out = sl.plan;
            out->kp.A = p.A;   // packed operands get their copies' addresses at run time
            out->kp.B = p.B;
            out->kp.C = p.C;
            out->kp.bias = p.bias;
            out->op[0].src = p.A;
            out->op[1].src = p.B;
            return true;
        }
    }
    return false;
}

void plan_remember(const PlanKey &k, const Plan &pl)
{
    PlanSlot &sl = t_plans[t_plan_next];
    t_plan_next = (t_plan_next + 1) % kPlanSlots;
    sl.used = true;
    sl.key = k;
    sl.plan = pl;
}

// A call without workspace: tg_gemm, tg_gemm_bias_relu, tg_gemm_ex (config_id
// -1) and tg_gemm_with_config.
tg_status run(int config_id, const Problem &p, hipStream_t stream)
{
    tg_status st = validate(p);
    if (st != TG_SUCCESS)
        return st;
    if (config_id < -1 || config_id >= kNumConfigs)
        return TG_ERROR_INVALID_VALUE;
    if (p.M == 0 || p.N == 0)
        return TG_SUCCESS;
    Plan pl;
    const PlanKey key = plan_key(p, config_id, 1, 0);
    if (!plan_cached(key, p, &pl)) {
        if ((st = plan_fixed(p, config_id, 1, 0, &pl)) != TG_SUCCESS)
            return st;
        if (!supports(kConfigs[pl.id], p))
            return TG_ERROR_UNSUPPORTED;
        plan_remember(key, pl);
    }
    int dev = 0;
    if ((st = check_problem_pointers(p, &dev)) != TG_SUCCESS)
        return st;
    return execute(pl, p, nullptr, stream);
}

// The plan of a workspace call (tg_gemm_ws, tg_select_plan): validation and
// the choice, no device calls.
tg_status plan_ws(const Problem &p, int config_id, int splits, size_t ws_bytes, Plan *pl)
{
    tg_status st = validate(p);
    if (st != TG_SUCCESS)
        return st;
    if (config_id < -1 || config_id >= kNumConfigs || splits < 0 || splits > kMaxSplits)
        return TG_ERROR_INVALID_VALUE;
    if (p.M == 0 || p.N == 0) {
        *pl = Plan{};
        return TG_SUCCESS;
    }
    const PlanKey key = plan_key(p, config_id, splits, ws_bytes);
    if (!plan_cached(key, p, pl)) {
        if (config_id < 0 && splits == 0)
            *pl = plan_auto(p, ws_bytes);
        else if ((st = plan_fixed(p, config_id, splits, ws_bytes, pl)) != TG_SUCCESS)
            return st;
        plan_remember(key, *pl);
    }
    return pl->ws_used() > ws_bytes ? TG_ERROR_WORKSPACE : TG_SUCCESS;
}

// A workspace call: ws of ws_bytes bytes (device memory of the current device,
// 16-byte aligned) or NULL with ws_bytes == 0.
tg_status run_ws(int config_id, int splits, const Problem &p, void *ws, size_t ws_bytes,
                 hipStream_t stream)
{
    if ((ws == nullptr && ws_bytes != 0) || !aligned(ws, 16))
        return TG_ERROR_INVALID_VALUE;
    Plan pl;
    tg_status st = plan_ws(p, config_id, splits, ws_bytes, &pl);
    if (st != TG_SUCCESS || p.M == 0 || p.N == 0)
        return st;
    int dev = 0;
    if ((st = check_problem_pointers(p, &dev)) != TG_SUCCESS)
        return st;
    if (pl.ws_used() > 0 && (st = check_span(ws, pl.ws_used(), dev)) != TG_SUCCESS)
        return st;
    return execute(pl, p, static_cast<char *>(ws), stream);
}

// ---- attention ----------------------------------------------------------------
constexpr int64_t kMaxRange = int64_t(1) << 31;

tg_status attention_args(const void *Q, const void *K, const void *V, void *O, float *lse,
                         int64_t B, int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                         const int64_t *qs, const int64_t *ks, const int64_t *vs,
                         const int64_t *os, float scale, int causal, tg::AttentionArgs *a)
{
    if (B < 0 || H < 1 || Hkv < 1 || H % Hkv || Lq < 0 || Lk < 0 || d < 1)
        return TG_ERROR_INVALID_VALUE;
    if (!qs || !ks || !vs || !os || !(scale == scale) || scale > 3.4e38f || scale < -3.4e38f ||
        (causal != 0 && causal != 1))
        return TG_ERROR_INVALID_VALUE;
    for (int i = 0; i < 3; i++)
        if (qs[i] < 0 || ks[i] < 0 || vs[i] < 0 || os[i] < 0)
            return TG_ERROR_INVALID_VALUE;
    if (B == 0 || Lq == 0)
        return TG_SUCCESS;   // nothing to compute
    if (!Q || !O || (Lk > 0 && (!K || !V)))
        return TG_ERROR_INVALID_VALUE;
    if (!aligned(Q, 2) || !aligned(K, 2) || !aligned(V, 2) || !aligned(O, 2) ||
        (lse && !aligned(lse, 4)))
        return TG_ERROR_INVALID_VALUE;
    // what this kernel supports: head dimension 64 or 128, 16-byte rows
    if (d != 64 && d != 128)
        return TG_ERROR_UNSUPPORTED;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
        return TG_ERROR_UNSUPPORTED;
    for (int i = 0; i < 3; i++)
        if (qs[i] % 8 || ks[i] % 8 || vs[i] % 8 || os[i] % 8)
            return TG_ERROR_UNSUPPORTED;
    if (B > kMaxDim || H > kMaxDim || Lq > kMaxDim || Lk > kMaxDim ||
        B * H * ((Lq + 127) / 128) > kMaxDim)
        return TG_ERROR_UNSUPPORTED;
    // the copies address a head's K / V rows with 32-bit offsets from the
    // tile's first row
    const int64_t k_bytes = Lk > 0 ? ((Lk - 1) * ks[2] + d) * 2 : 0;
    const int64_t v_bytes = Lk > 0 ? ((Lk - 1) * vs[2] + d) * 2 : 0;
    if (k_bytes >= kMaxRange || v_bytes >= kMaxRange || (Lk + 64) * ks[2] * 2 >= kMaxRange ||
        (Lk + 64) * vs[2] * 2 >= kMaxRange)
        return TG_ERROR_UNSUPPORTED;
    memset(a, 0, sizeof(*a));
    a->Q = Q;
    a->K = K;
    a->V = V;
    a->O = O;
    a->lse = lse;
    a->B = (int)B;
    a->H = (int)H;
    a->Hkv = (int)Hkv;
    a->Lq = (int)Lq;
    a->Lk = (int)Lk;
    a->d = (int)d;
    for (int i = 0; i < 3; i++) {
        a->qs[i] = qs[i];
        a->ks[i] = ks[i];
        a->vs[i] = vs[i];
        a->os[i] = os[i];
    }
    a->k_bytes = (uint32_t)k_bytes;
    a->v_bytes = (uint32_t)v_bytes;
    a->scale = scale;
    a->causal = causal;
    return TG_SUCCESS;
}

}  // namespace

extern "C" {

tg_status tg_attention_fwd(const void *Q, const void *K, const void *V, void *O, float *lse,
                           int64_t B, int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                           const int64_t *q_strides, const int64_t *k_strides,
                           const int64_t *v_strides, const int64_t *o_strides, float scale,
                           int causal, hipStream_t stream)
{
    tg::AttentionArgs a;
    memset(&a, 0, sizeof(a));
    tg_status st = attention_args(Q, K, V, O, lse, B, H, Hkv, Lq, Lk, d, q_strides, k_strides,
                                  v_strides, o_strides, scale, causal, &a);
    if (st != TG_SUCCESS || B == 0 || Lq == 0)
        return st;
    int dev = 0;
    if ((st = check_device(&dev)) != TG_SUCCESS)
        return st;
    // every element read or written lies inside its allocation
    auto extent = [d](const int64_t *s, int64_t b, int64_t h, int64_t l) {
        return 2 * (uint64_t)((b - 1) * s[0] + (h - 1) * s[1] + (l - 1) * s[2] + d);
    };
    if ((st = check_span(Q, extent(q_strides, B, H, Lq), dev)) != TG_SUCCESS ||
        (st = check_span(O, extent(o_strides, B, H, Lq), dev)) != TG_SUCCESS ||
        (Lk > 0 && ((st = check_span(K, extent(k_strides, B, Hkv, Lk), dev)) != TG_SUCCESS ||
                    (st = check_span(V, extent(v_strides, B, Hkv, Lk), dev)) != TG_SUCCESS)) ||
        (st = check_span(lse, 4 * (uint64_t)(B * H * Lq), dev)) != TG_SUCCESS)
        return st;
    (void)hipGetLastError();
    return tg::launch_attention(a, stream) == hipSuccess ? TG_SUCCESS : TG_ERROR_LAUNCH;
}


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
    case TG_ERROR_FILE: return "TG_ERROR_FILE: file cannot be opened or read";
    case TG_ERROR_WORKSPACE: return "TG_ERROR_WORKSPACE: the plan needs more workspace than the call provides";
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
    out->whole_k = c.whole_k;
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

tg_status tg_tuning_load(const char *path, int *loaded, int *skipped, int *error_line)
{
    ensure_env_cache();
    if (path == nullptr) {
        if (error_line)
            *error_line = 0;
        return TG_ERROR_INVALID_VALUE;
    }
    auto t = std::make_shared<TuneTable>();
    const tg_status st = read_tuning_file(path, t.get(), loaded, skipped, error_line);
    if (st == TG_SUCCESS)
        publish(std::move(t));
    return st;
}

tg_status tg_tuning_clear(void)
{
    ensure_env_cache();
    publish(nullptr);
    return TG_SUCCESS;
}

int tg_tuning_count(void)
{
    ensure_env_cache();
    std::lock_guard<std::mutex> lk(g_tune_mu);
    return g_tune ? (int)g_tune->size() : 0;
}

size_t tg_splitk_workspace_bytes(int64_t M, int64_t N, int splits)
{
    if (M <= 0 || N <= 0 || splits <= 1 || splits > kMaxSplits)
        return 0;
    return (size_t)splits * (size_t)M * (size_t)N * 4;
}

tg_status tg_gemm_ws(int config_id, int splits, tg_op op_a, tg_op op_b, const void *A,
                     const void *B, const float *bias, void *C, int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc, tg_dtype c_dtype, void *workspace,
                     size_t workspace_bytes, hipStream_t stream)
{
    return run_ws(config_id, splits,
                  Problem{A, B, bias, C, M, N, K, lda, ldb, ldc, c_dtype, bias != nullptr, op_a,
                          op_b},
                  workspace, workspace_bytes, stream);
}

tg_status tg_select_plan(tg_op op_a, tg_op op_b, const void *A, const void *B,
                         const float *bias, const void *C, int64_t M, int64_t N, int64_t K,
                         int64_t lda, int64_t ldb, int64_t ldc, tg_dtype c_dtype,
                         size_t workspace_bytes, int *config_id, int *splits, int *packed,
                         size_t *workspace_used)
{
    if (config_id == nullptr || splits == nullptr || packed == nullptr || workspace_used == nullptr)
        return TG_ERROR_INVALID_VALUE;
    *config_id = -1;
    *splits = 1;
    *packed = 0;
    *workspace_used = 0;
    Plan pl;
    const tg_status st = plan_ws(Problem{A, B, bias, const_cast<void *>(C), M, N, K, lda, ldb,
                                         ldc, c_dtype, bias != nullptr, op_a, op_b},
                                 -1, 0, workspace_bytes, &pl);
    if (st != TG_SUCCESS)
        return st;
    *config_id = pl.id;
    *splits = (int)pl.slices;
    *packed = (pl.pack[0] ? 1 : 0) | (pl.pack[1] ? 2 : 0);
    *workspace_used = pl.ws_used();
    return TG_SUCCESS;
}

tg_status tg_mfma_ceiling(int mfma, const void *operands, float *sink, int64_t iters,
                          int64_t workgroups, hipStream_t stream)
{
    // iters * workgroups is capped at 2^32 (about ten seconds of matrix-core
    // work) so that one call cannot hold the device for minutes
    if ((mfma != 16 && mfma != 32 && mfma != 64) || operands == nullptr || sink == nullptr ||
        iters < 2 ||
        iters > (int64_t(1) << 30) || (iters & 1) || workgroups < 1 ||
        workgroups > (int64_t(1) << 20) || iters * workgroups > (int64_t(1) << 32))
        return TG_ERROR_INVALID_VALUE;
    if (!aligned(operands, 16) || !aligned(sink, 4))
        return TG_ERROR_INVALID_VALUE;
    int dev = 0;
    tg_status st;
    // both buffers must lie inside their allocations
    if ((st = check_device(&dev)) != TG_SUCCESS ||
        (st = check_span(operands, TG_CEILING_OPERAND_BYTES, dev)) != TG_SUCCESS ||
        (st = check_span(sink, (uint64_t)workgroups * 512 * sizeof(float), dev)) != TG_SUCCESS)
        return st;
    (void)hipGetLastError();
    return tg::launch_mfma_ceiling(mfma, operands, sink, (int)iters, (int)workgroups, stream) ==
                   hipSuccess
               ? TG_SUCCESS
               : TG_ERROR_LAUNCH;
}

const char *tg_version(void) { return "tg 0.5.0 (gfx950)"; }

}  // extern "C"
