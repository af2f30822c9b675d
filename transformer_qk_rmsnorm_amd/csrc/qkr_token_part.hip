// One instantiation unit of the token-tile QK RMSNorm + RoPE kernels: every
// variant with QKR_TOKEN_L lanes per row and QKR_EAGER numerics (the build
// compiles this file once per pair of values).
#include "qkr_rope_kernel.hpp"

#if !defined(QKR_TOKEN_L) || !defined(QKR_EAGER)
#error "build with -DQKR_TOKEN_L=<lanes per row> -DQKR_EAGER=<0 or 1>"
#endif

namespace qkr {

template <>
NormRopeFn pick_norm_rope_token<QKR_TOKEN_L, (QKR_EAGER != 0)>(int32_t dtype, int rope, int32_t pairing, bool nt)
{
    return dtype == kBF16 ? pick_token_rope<BF16, QKR_TOKEN_L, (QKR_EAGER != 0)>(rope, pairing, nt)
                          : pick_token_rope<F32, QKR_TOKEN_L, (QKR_EAGER != 0)>(rope, pairing, nt);
}

}  // namespace qkr
