// One instantiation unit of the QK RMSNorm + RoPE kernels: every variant
// with QKR_LPR lanes per row and QKR_EAGER numerics (the build compiles this
// file once per pair of values).
#include "qkr_rope_kernel.hpp"

#if !defined(QKR_LPR) || !defined(QKR_EAGER)
#error "build with -DQKR_LPR=<lanes per row> -DQKR_EAGER=<0 or 1>"
#endif

namespace qkr {

template <>
NormRopeFn pick_norm_rope<QKR_LPR, (QKR_EAGER != 0)>(int32_t dtype, int rope, int32_t pairing, bool nt, bool stage,
                                                     int np)
{
    return dtype == kBF16 ? pick_rope<BF16, QKR_LPR, (QKR_EAGER != 0)>(rope, pairing, nt, stage, np)
                          : pick_rope<F32, QKR_LPR, (QKR_EAGER != 0)>(rope, pairing, nt, stage, np);
}

}  // namespace qkr
