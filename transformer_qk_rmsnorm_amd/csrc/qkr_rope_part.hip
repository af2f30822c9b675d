// One instantiation unit of the QK RMSNorm + RoPE kernels: every variant
// with QKR_LPR lanes per row (the build compiles this file once per value).
#include "qkr_rope_kernel.hpp"

#ifndef QKR_LPR
#error "build with -DQKR_LPR=<lanes per row>"
#endif

namespace qkr {

template <>
NormRopeFn pick_norm_rope<QKR_LPR>(int32_t dtype, int rope, int32_t pairing, bool nt, bool stage, int np)
{
    return dtype == kBF16 ? pick_rope<BF16, QKR_LPR>(rope, pairing, nt, stage, np)
                          : pick_rope<F32, QKR_LPR>(rope, pairing, nt, stage, np);
}

}  // namespace qkr
