// The kernel side of libtg as the host code sees it, for the sanitizer build
// of the host code (tests/sanitize/host_driver.cpp), which runs without a
// GPU and so never launches: the configuration table, built from the same
// list as the library's (tg_config_list.inc) with the same names and LDS
// sizes, and launch functions that report an error.  test_sanitize_cpu.py
// checks the table against the built library's, row by row.
#include <hip/hip_runtime_api.h>

#include "tg_attention.h"
#include "tg_ceiling.h"
#include "tg_kernels.h"
#include "tg.h"
#include "tg_pack.h"

namespace tg {

// LDS of a configuration: STAGES buffers of a BM x BK and a BK x BN tile.
#define TG_STUB_LDS(BM, BN, BK, ST, ES) ((ST) * ((BM) * (BK) + (BK) * (BN)) * (ES))
#define TG_CONFIG_ROW(ID, BM, BN, BK, WM, WN, ST, MI, KIND, SCH, OPS, ES)                          \
    {ID, BM, BN, BK, ST, WM, WN, MI, (KIND) == 2, TG_STUB_LDS(BM, BN, BK, ST, ES), OPS, ES,        \
     (SCH) == 3,                                                                                 \
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
#undef TG_CONFIG_ROW
const int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

static hipError_t no_launch(const Params &, bool, bool, hipStream_t)
{
    return hipErrorInvalidDeviceFunction;
}

LaunchFn config_launch(int id) { return id >= 0 && id < kNumConfigs ? &no_launch : nullptr; }

hipError_t launch_splitk_reduce(const ReduceParams &, OutKind, hipStream_t)
{
    return hipErrorInvalidDeviceFunction;
}

hipError_t launch_pack(const PackOperand *, int, hipStream_t) { return hipErrorInvalidDeviceFunction; }

hipError_t launch_attention(const AttentionArgs &, hipStream_t) { return hipErrorInvalidDeviceFunction; }

hipError_t launch_mfma_ceiling(int, const void *, float *, int, int, hipStream_t)
{
    return hipErrorInvalidDeviceFunction;
}

}  // namespace tg

// The static-workspace entry point lives with its device array in
// tg_static.hip; without a device it would stop at the device check.
extern "C" tg_status tg_gemm_ws_static(int, int, tg_op, tg_op, const void *, const void *,
                                       const float *, void *, int64_t, int64_t, int64_t, int64_t,
                                       int64_t, int64_t, tg_dtype, hipStream_t)
{
    return TG_ERROR_UNSUPPORTED;
}
