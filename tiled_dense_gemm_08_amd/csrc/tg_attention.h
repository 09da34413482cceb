// tg_attention.h — internal interface between the host dispatcher
// (tg_api.cpp) and the fused attention kernel (tg_attention.hip).  Not
// installed, not part of the ABI.
#ifndef TG_ATTENTION_H
#define TG_ATTENTION_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tg {

// Fused attention forward (tg_attention.hip).  Element (b, h, i, c) of Q is
// Q[b qs[0] + h qs[1] + i qs[2] + c]; K and V likewise with their Hkv heads;
// O like Q.  k_bytes / v_bytes: bytes from a head's first K / V row to the end
// of its last (the copies' descriptor range).
struct AttentionArgs {
    const void *Q, *K, *V;
    void *O;
    float *lse;
    int B, H, Hkv, Lq, Lk, d;
    int64_t qs[3], ks[3], vs[3], os[3];
    uint32_t k_bytes, v_bytes;
    float scale;
    int causal;
};

hipError_t launch_attention(const AttentionArgs &a, hipStream_t s);

}  // namespace tg

#endif
