// tg_ceiling.h — internal interface between the host side (tg_api.cpp) and
// the matrix-core rate kernel (tg_ceiling.hip).  Not installed, not part of
// the ABI.
#ifndef TG_CEILING_H
#define TG_CEILING_H

#include <hip/hip_runtime_api.h>

namespace tg {

// `workgroups` workgroups of 256 threads; thread t of every workgroup reads
// the 512 bytes at operands + 512 t (131072 bytes in all) and writes one
// float to sink[256 * workgroup + t].  mfma: 16 (16x16x32) or 32 (32x32x16);
// iters > 0 and even.  Arguments are validated by the caller.
hipError_t launch_mfma_ceiling(int mfma, const void *operands, float *sink, int iters,
                               int workgroups, hipStream_t s);

}  // namespace tg

#endif
