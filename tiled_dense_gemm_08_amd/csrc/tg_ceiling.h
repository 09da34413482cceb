// tg_ceiling.h — internal interface between the host side (tg_api.cpp) and
// the matrix-core rate kernel (tg_ceiling.hip).  Not installed, not part of
// the ABI.
#ifndef TG_CEILING_H
#define TG_CEILING_H

#include <hip/hip_runtime_api.h>

namespace tg {

// `workgroups` workgroups of 512 threads; every thread reads 16-byte chunks
// of the 131072-byte operand buffer (A fragments from its first half, B
// fragments from its second) and writes one float to sink[512 * workgroup +
// t].  mfma: 16 (16x16x32 fp16), 32 (32x32x16 fp16) or 64 (16x16x64 int8);
// iters > 0 and even.  Arguments are validated by the caller.
hipError_t launch_mfma_ceiling(int mfma, const void *operands, float *sink, int iters,
                               int workgroups, hipStream_t s);

}  // namespace tg

#endif
