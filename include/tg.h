/*
 * tg.h — C ABI of libtg.so: a tiled fp16 matrix multiply for AMD Instinct
 * MI355X (gfx950), with an optional fused bias + ReLU epilogue.
 *
 * Operation (lqnn.cn TileLang walkthrough, section 2.1, the tiled matmul
 * listing, and section 4.2, the runnable FP16-input / FP32-accumulate GEMM;
 * codechina.net TileLang article, section 3.2, the variant with float32 C):
 *     C[i][j] = sum_{k<K} A[i][k] * B[k][j]
 * with fp16 A and B, fp32 accumulation and C stored as fp16 or fp32.
 * Fused variant (xdnf.cn TileLang article, section 4.2, GEMM + bias + ReLU):
 *     C[i][j] = max(sum_k A[i][k] * B[k][j] + bias[j], 0)
 *
 * Layout: every matrix is row-major.  A is M x K with leading dimension lda
 * (element (i,k) at A[i*lda + k]); B is K x N with ldb; C is M x N with ldc.
 * Leading dimensions are in elements.  bias is fp32, length N, indexed by the
 * output column.
 *
 * Ownership: the caller owns every buffer.  A, B, C and bias must be device
 * memory of the current HIP device (hipMalloc, or a framework allocation on
 * that device).  The library never allocates device memory: the calls that
 * can use more memory than their operands (tg_gemm_ws) take a workspace the
 * caller owns.  Apart from the read-only tuning cache, the library keeps no
 * state between calls and is safe to call from several host threads.  Calls
 * are asynchronous on `stream` (NULL = the default stream): the buffers must
 * stay alive, and C must not be read, until the stream has passed the launch.
 * C must not alias A, B or bias.
 *
 * Errors: arguments are validated on the host before any device work; on an
 * error nothing is launched and C is untouched.  Execution faults surface at
 * the caller's next synchronisation.
 *   TG_ERROR_INVALID_VALUE     negative M/N/K; lda < K, ldb < N or ldc < N
 *                              (the stored widths for tg_gemm_ex);
 *                              a NULL pointer when the call has work to do; a
 *                              NULL bias in the fused call; an unknown dtype;
 *                              a pointer not aligned to its element size; an
 *                              unknown config id; a buffer whose elements run
 *                              past the end of the allocation that holds it
 *                              (A over its (rows - 1) * lda + cols stored
 *                              elements, B and C likewise, bias over N; checked
 *                              with hipMemGetAddressRange, i.e. against the
 *                              whole hipMalloc block of a pooled allocation)
 *   TG_ERROR_NOT_DEVICE_MEMORY a pointer that is host or unregistered memory,
 *                              or device memory of another device (a host
 *                              pointer would otherwise read as garbage or an
 *                              empty result instead of failing -- the pitfall
 *                              noted in the lqnn.cn walkthrough, section 5.2)
 *   TG_ERROR_UNSUPPORTED       the current device is not gfx950, or an operand
 *                              spans 2 GiB or more (32-bit buffer offsets)
 *   TG_ERROR_LAUNCH            the HIP runtime rejected the kernel launch
 *   TG_ERROR_WORKSPACE         (tg_gemm_ws) the plan the caller named needs
 *                              more workspace than the call provides
 *
 * Edge cases: M == 0 or N == 0 is a successful no-op.  K == 0 writes zeros
 * (the empty sum), or relu(bias[j]) in the fused call.
 */
#ifndef TG_H
#define TG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are int-sized.  Compiled as C++ they have int as their
 * fixed underlying type, so that any int a caller passes is a valid value
 * for the library to receive and reject (without a fixed type, a C++ enum
 * holds only the values its enumerators' bits span). */
#ifdef __cplusplus
#define TG_ENUM(name) enum name : int
#else
#define TG_ENUM(name) enum name
#endif

/* Output type.  TG_DTYPE_I32 selects the int8 product: A and B then hold
 * int8 values and C = op(A).op(B) is accumulated and stored in int32 (exact:
 * K is limited to 131072 so that no partial sum leaves int32). */
typedef TG_ENUM(tg_dtype_e) { TG_DTYPE_F16 = 1, TG_DTYPE_F32 = 2, TG_DTYPE_I32 = 3 } tg_dtype;

/* Operand orientation for tg_gemm_ex: TG_OP_N uses the stored matrix as is,
 * TG_OP_T uses its transpose. */
typedef TG_ENUM(tg_op_e) { TG_OP_N = 0, TG_OP_T = 1 } tg_op;

typedef TG_ENUM(tg_status_e) {
    TG_SUCCESS = 0,
    TG_ERROR_INVALID_VALUE = 1,
    TG_ERROR_NOT_DEVICE_MEMORY = 2,
    TG_ERROR_UNSUPPORTED = 3,
    TG_ERROR_LAUNCH = 4,
    TG_ERROR_FILE = 5,           /* tg_tuning_load: the file cannot be opened or read */
    TG_ERROR_WORKSPACE = 6       /* tg_gemm_ws: workspace too small for the named plan */
} tg_status;

/* C = A.B (overwrites C; no alpha/beta scaling).  A, B: fp16; C: c_dtype. */
tg_status tg_gemm(const void *A, const void *B, void *C,
                  int64_t M, int64_t N, int64_t K,
                  int64_t lda, int64_t ldb, int64_t ldc,
                  tg_dtype c_dtype, hipStream_t stream);

/* C = max(A.B + bias[col], 0) (overwrites C).  bias: fp32[N], required. */
tg_status tg_gemm_bias_relu(const void *A, const void *B, const float *bias, void *C,
                            int64_t M, int64_t N, int64_t K,
                            int64_t lda, int64_t ldb, int64_t ldc,
                            tg_dtype c_dtype, hipStream_t stream);

/* C = op(A).op(B), or max(op(A).op(B) + bias[col], 0) when bias != NULL
 * (overwrites C).  The operand layouts of the backward products of a linear
 * layer (codechina.net TileLang article, section 5.1: dA = G.B^T, dB = A^T.G;
 * xdnf.cn article, section 4.3: the layout decides the access path):
 *   op_a == TG_OP_N: A is M x K row-major, lda >= K;
 *   op_a == TG_OP_T: A is stored K x M row-major (element (i,k) of op(A) at
 *                    A[k*lda + i]), lda >= M;
 *   op_b == TG_OP_N: B is K x N row-major, ldb >= N;
 *   op_b == TG_OP_T: B is stored N x K row-major (element (k,j) of op(B) at
 *                    B[j*ldb + k]), ldb >= K.
 * C is M x N row-major with ldc >= N.  Same ownership, validation and errors
 * as tg_gemm; an op outside {TG_OP_N, TG_OP_T} is TG_ERROR_INVALID_VALUE.
 * tg_gemm(...) equals tg_gemm_ex(TG_OP_N, TG_OP_N, A, B, NULL, C, ...).
 * c_dtype == TG_DTYPE_I32: int8 A and B, int32 C (the quantized variant the
 * pwwt.cn article names as a next step, section 5.3; exact integer
 * arithmetic); bias must be NULL (TG_ERROR_INVALID_VALUE otherwise) and
 * K > 131071 is TG_ERROR_UNSUPPORTED. */
tg_status tg_gemm_ex(tg_op op_a, tg_op op_b, const void *A, const void *B,
                     const float *bias, void *C,
                     int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc,
                     tg_dtype c_dtype, hipStream_t stream);

/* ---- the dispatcher with a caller-owned workspace --------------------------
 * The same product as tg_gemm_ex, run by a plan that may use device memory
 * beyond the operands: a workspace the caller passes in.  Two techniques use
 * it, alone or together:
 *
 *  K slices (split-K).  For problems with few output tiles and a long K (M*N
 *  small next to the 256 CUs, K large) one workgroup per output tile leaves
 *  most of the chip idle.  K is cut into `slices` slices of k_split elements
 *  (K/slices rounded up to the kernel's K step; fewer slices when K is short);
 *  every slice's product runs as its own set of workgroups, each writing an
 *  fp32 (int32 for int8 operands) partial product of C to the workspace, and
 *  a second kernel on the same stream sums the partials in slice order, adds
 *  the bias, applies ReLU and converts to C's type.  The order is fixed, so a
 *  result is reproducible; it may differ from the unsliced call's by fp32
 *  rounding (for integer inputs and int8 operands it is exact and equal).
 *  Partials take slices * M * N * 4 bytes.
 *
 *  Packed operands.  The direct configurations copy 16-byte chunks of A and
 *  B straight to LDS; an operand whose base is not 16-byte aligned, or whose
 *  leading dimension or row length is not a multiple of 16 bytes, is
 *  otherwise read by a register-staged configuration (what tg_gemm_ex does).
 *  The plan may instead copy such an operand into the workspace in a packed
 *  layout -- the same stored rows, each padded with zeros to a multiple of
 *  16 bytes, which is also the copy's leading dimension -- and run a direct
 *  configuration on the copy with K rounded up to a whole chunk.  Zeros added
 *  to a sum change nothing (on integer inputs the result is bit-identical).
 *  A copy takes rows * (cols rounded up to 16 bytes) bytes, rounded up to 256.
 *
 * The product is the one defined at the top of this file; only the grouping
 * of the K sum changes.  Workspace layout: the copies first, then the
 * partials.
 *
 * config_id: -1 = the dispatcher's choice, else that configuration.
 * splits:    0 = chosen: with config_id == -1, the plan with the least
 *            modelled time among the operands as passed (unsliced, or in 2..32
 *            slices) and packed copies (unsliced or sliced) whose workspace
 *            fits workspace_bytes (a tuning-cache record for the exact problem
 *            is run as recorded: unpacked, unsliced); with a named
 *            configuration, the slice count only (never packed);
 *            1 = unsliced and unpacked (the workspace is not used);
 *            2..64 = that many slices of the operands as passed (never
 *            packed).
 * workspace: device memory of the current device, 16-byte aligned, not
 *            overlapping A, B, C or bias; NULL only with workspace_bytes 0.
 *            Owned by the caller, who keeps it alive and does not reuse it
 *            until the stream has passed the call: calls that share a
 *            workspace must be ordered (same stream, or synchronised).  The
 *            library writes every workspace byte it reads in the same call,
 *            so no clearing is needed.
 * Errors: as tg_gemm_ex; additionally TG_ERROR_INVALID_VALUE for splits
 * outside 0..64, an unknown config_id, a NULL workspace with nonzero
 * workspace_bytes or one not 16-byte aligned; TG_ERROR_WORKSPACE when the
 * named slice count needs more than workspace_bytes; TG_ERROR_UNSUPPORTED when
 * the named configuration cannot run the problem; TG_ERROR_NOT_DEVICE_MEMORY
 * or TG_ERROR_INVALID_VALUE for a workspace that is not device memory of the
 * current device or whose used part runs past its allocation. */
tg_status tg_gemm_ws(int config_id, int splits, tg_op op_a, tg_op op_b, const void *A,
                     const void *B, const float *bias, void *C,
                     int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc, tg_dtype c_dtype,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): tg_gemm_ws
 * with the library's own workspace, a device array of TG_STATIC_SCRATCH_BYTES
 * in place of the caller's, so the call allocates nothing and the caller
 * passes only its inputs and outputs.  Each GPU the library runs on holds its
 * own copy of the array until the process ends.  Arguments, plans and errors
 * as tg_gemm_ws with workspace_bytes = TG_STATIC_SCRATCH_BYTES: the
 * dispatcher's plans (config_id -1, splits 0) are those whose workspace fits
 * the array, and a named plan that needs more is rejected with
 * TG_ERROR_WORKSPACE before anything is launched.
 * Every call on one GPU uses that GPU's single array: calls that overlap on
 * one GPU (on different streams without ordering, or from several host
 * threads on different streams) race and give wrong results; calls ordered on
 * one stream do not.  The array keeps the last call's contents; every byte a
 * call reads it has written first, so nothing needs clearing.
 * TG_ERROR_UNSUPPORTED when there is no current device, TG_ERROR_LAUNCH when
 * the runtime cannot give the array's device address. */
#define TG_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
tg_status tg_gemm_ws_static(int config_id, int splits, tg_op op_a, tg_op op_b, const void *A,
                            const void *B, const float *bias, void *C,
                            int64_t M, int64_t N, int64_t K,
                            int64_t lda, int64_t ldb, int64_t ldc, tg_dtype c_dtype,
                            hipStream_t stream);

/* Partial-product bytes of `splits` K slices: splits * M * N * 4 (0 if
 * splits <= 1 or M, N <= 0; 0 also for splits > 64, which the calls reject). */
size_t tg_splitk_workspace_bytes(int64_t M, int64_t N, int splits);

/* What tg_gemm_ws(-1, 0, ..., workspace_bytes, ...) runs: *config_id the
 * configuration (-1 for an empty problem), *splits the slice count (1:
 * unsliced), *packed a bit mask of the operands copied first (1: A, 2: B) and
 * *workspace_used the workspace bytes the plan uses (<= workspace_bytes).
 * With workspace_bytes = SIZE_MAX, *workspace_used is the workspace the
 * dispatcher's fastest plan needs.  Touches no device state; returns the
 * argument errors the call would (TG_ERROR_INVALID_VALUE, also for NULL
 * outputs). */
tg_status tg_select_plan(tg_op op_a, tg_op op_b, const void *A, const void *B,
                         const float *bias, const void *C, int64_t M, int64_t N, int64_t K,
                         int64_t lda, int64_t ldb, int64_t ldc, tg_dtype c_dtype,
                         size_t workspace_bytes, int *config_id, int *splits, int *packed,
                         size_t *workspace_used);

/* ---- fused attention (forward) -------------------------------------------
 * O = softmax(scale * Q K^T [+ causal mask]) V for every batch b < B and
 * query head h < H, computed block by block with the softmax folded in online
 * (lqnn.cn TileLang walkthrough, section 3.2; xdnf.cn article, section 3.2):
 *   s_ij  = scale * sum_c Q[b][h][i][c] K[b][hk][j][c]   (hk = h / (H / Hkv))
 *   O[b][h][i][c] = sum_j softmax_j(s_ij) V[b][hk][j][c]
 *   lse[b][h][i]  = log sum_j exp(s_ij)            (natural log)
 * over the visible keys: j < Lk and, with causal = 1, j <= i + (Lk - Lq)
 * (the mask aligned at the bottom right: with Lq == Lk, j <= i).  A query
 * that sees no key gets O = 0 and lse = -inf.  scale may have either sign;
 * scale == 0 gives every visible key the same weight, exactly.
 *
 * Q, K, V, O: fp16; scores, softmax and the weighted sum in fp32, the
 * softmax weights rounded to fp16 for the second product.  Layout: element
 * (b, h, i, c) of Q is Q[b * q_strides[0] + h * q_strides[1] + i *
 * q_strides[2] + c] (strides in elements, the head dimension contiguous);
 * K and V likewise with their Hkv heads; O like Q.  [B, H, L, d] and
 * [B, L, H, d] are both such layouts.  lse: NULL, or fp32 [B][H][Lq] dense.
 * O must not overlap Q, K, V or lse.  Asynchronous on `stream`.
 *
 * Errors: TG_ERROR_INVALID_VALUE for negative sizes or strides, H not a
 * multiple of Hkv, NULL strides or required pointers (K, V may be NULL when
 * Lk == 0), a non-finite scale, causal not 0 or 1, or a pointer not aligned
 * to its element; TG_ERROR_UNSUPPORTED for d other than 64 or 128, Q, K, V
 * or O not 16-byte aligned, a stride not a multiple of 8 elements, or a
 * head's K or V rows spanning 2 GiB or more; TG_ERROR_NOT_DEVICE_MEMORY and
 * TG_ERROR_LAUNCH as for the GEMM.  B == 0 or Lq == 0 is a successful no-op. */
tg_status tg_attention_fwd(const void *Q, const void *K, const void *V, void *O, float *lse,
                           int64_t B, int64_t H, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                           const int64_t *q_strides, const int64_t *k_strides,
                           const int64_t *v_strides, const int64_t *o_strides,
                           float scale, int causal, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char *tg_status_string(tg_status s);

/* ---- tuning and test entry points ---------------------------------------
 * The kernel configurations (block tile, K step, pipeline stages, waves per
 * workgroup, load path) compiled into the library.  The dispatcher above
 * picks one per call (lqnn.cn walkthrough, sections 2.3 and 5.3: search block
 * sizes and stages on the real device, record the best per shape, read the
 * record at run time), trying in order
 *   1. the run-time tuning cache below (exact shape, orientation, C dtype and
 *      fused flag),
 *   2. a compiled table of exact shapes,
 *   3. a compiled cost model: per configuration, the time of a full and of a
 *      lone round of workgroups as a function of K, fitted to on-device
 *      timings; the configuration with the least predicted time wins,
 *   4. the register-staged kernels, which take any alignment,
 * and at each step uses the configuration only if it can run the problem
 * (tg_config_supports).  tg_gemm, tg_gemm_bias_relu and tg_gemm_ex run that
 * configuration on the operands as passed; tg_gemm_ws may also slice K or
 * pack operands (above). */

typedef struct {
    int id;
    int block_m, block_n, block_k;   /* workgroup output tile and K step */
    int stages;                      /* LDS ring depth of the K pipeline */
    int waves_m, waves_n;            /* wave64 grid inside the workgroup */
    int mfma;                        /* MFMA block edge: 16 (v_mfma_f32_16x16x32_f16)
                                        or 32 (v_mfma_f32_32x32x16_f16) */
    int direct_lds;                  /* 1: 16-byte global->LDS DMA loads (aligned
                                        operands only); 0: register-staged loads
                                        with per-element bounds (any alignment) */
    int lds_bytes;                   /* LDS per workgroup */
    int ops;                         /* orientations compiled: bit (1 << (2*op_a + op_b)) */
    int elem_bytes;                  /* operand element: 2 fp16, 1 int8 (int32 C) */
    int whole_k;                     /* 1: runs only K that is a multiple of block_k
                                        (tg_config_supports answers 0 otherwise) */
    const char *name;                /* static string */
} tg_config_desc;

/* Number of configurations; ids are 0 .. tg_num_configs()-1. */
int tg_num_configs(void);

/* Describe configuration `id`; TG_ERROR_INVALID_VALUE for an unknown id. */
tg_status tg_config_info(int id, tg_config_desc *out);

/* Whether configuration `id` can run this problem (orientation compiled;
 * alignment and leading-dimension requirements of its load path; K in whole
 * K steps where whole_k is set): 1 yes,
 * 0 no, -1 invalid arguments.  Arguments as for tg_gemm_ex. */
int tg_config_supports(int id, tg_op op_a, tg_op op_b, const void *A, const void *B,
                       const float *bias, const void *C, int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc, tg_dtype c_dtype);

/* The configuration id tg_gemm_ex runs for these arguments, or -1 for
 * invalid arguments.  Touches no device state. */
int tg_select_config(tg_op op_a, tg_op op_b, const void *A, const void *B, const float *bias,
                     const void *C, int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc, tg_dtype c_dtype);

/* Run one specific configuration; otherwise as tg_gemm_ex.  Additionally
 * TG_ERROR_INVALID_VALUE for an unknown id and TG_ERROR_UNSUPPORTED when the
 * configuration cannot run this problem (see tg_config_supports). */
tg_status tg_gemm_with_config(int config_id, tg_op op_a, tg_op op_b, const void *A,
                              const void *B, const float *bias, void *C,
                              int64_t M, int64_t N, int64_t K,
                              int64_t lda, int64_t ldb, int64_t ldc,
                              tg_dtype c_dtype, hipStream_t stream);

/* ---- run-time tuning cache ------------------------------------------------
 * Exact-shape records written by the on-device sweep (the sweep's --tune
 * mode) and read, never written, by the library: the offline-tune /
 * online-lookup scheme of the lqnn.cn walkthrough, section 5.3.  File format
 * (text): the first line is exactly "tg-tuning 1"; blank lines and lines
 * starting with '#' are ignored; every other line is one record of ten
 * whitespace-separated fields
 *     M N K op_a op_b c_dtype fused config name tflops
 * with op_a, op_b in {N, T}, c_dtype in {f16, f32, i32}, fused in {0, 1}
 * (i32 only with 0), config a configuration id, name that configuration's
 * name (tg_config_desc.name) and tflops the measured rate (informational).
 * A record whose id names another kernel than `name` in this library, or a
 * kernel that cannot serve its orientation or C dtype, is stale: it is
 * skipped and counted.  A later record for the same key replaces an earlier
 * one.  At dispatch a cached configuration that cannot run the actual
 * pointers or leading dimensions (alignment) is passed over.
 *
 * If the environment variable TG_TUNING_FILE names a file, it is loaded once,
 * before the first call that reads or changes the cache; if it does not
 * load, the cache starts empty and one line on stderr says why.
 *
 * The cache is process-wide and safe to use from several threads: a load
 * builds a new table and replaces the old one whole, so each GEMM call sees
 * either of them.  The tables are host memory. */

/* Replace the cache with the records of the file at `path`.  On success
 * *loaded receives the number of distinct keys now cached and *skipped the
 * number of stale records.  On failure the cache is unchanged and
 * *error_line receives the 1-based line that could not be parsed (0 for an
 * I/O error).  Any of the three out pointers may be NULL.
 * Errors: TG_ERROR_INVALID_VALUE (NULL path; missing or wrong first line;
 * a malformed record or an over-long line; more than 2^20 records),
 * TG_ERROR_FILE (cannot open or read). */
tg_status tg_tuning_load(const char *path, int *loaded, int *skipped, int *error_line);

/* Empty the cache (the compiled tables still apply).  Always TG_SUCCESS. */
tg_status tg_tuning_clear(void);

/* Number of keys in the cache. */
int tg_tuning_count(void);

/* Library version string (static). */
const char *tg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TG_H */
