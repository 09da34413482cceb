// tg_pack.h — internal interface between the host dispatcher (tg_api.cpp)
// and the operand pack kernel (tg_pack.hip).  Not installed, not part of the
// ABI.
#ifndef TG_PACK_H
#define TG_PACK_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tg {

// One stored matrix to copy into a packed, zero-padded layout: `rows` stored
// rows of `cols` elements (es bytes each) at leading dimension `ld` become
// `rows` rows of `cols_p` elements, leading dimension cols_p, at `dst`
// (16-byte aligned; cols_p * es a multiple of 16 and cols_p >= cols).
// Elements cols .. cols_p - 1 of every row are zeros.
struct PackOperand {
    const void *src;
    void *dst;
    int64_t rows, cols, ld, cols_p;
    int es;
};

// Packs one or two operands in one launch (n = 1 or 2).  Every 16-byte chunk
// of a packed row is one thread's job; chunk counts stay below 2^31.
hipError_t launch_pack(const PackOperand *ops, int n, hipStream_t s);

}  // namespace tg

#endif
