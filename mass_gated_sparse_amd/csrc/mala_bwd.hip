// MALA backward, bf16 inputs, head dim 128 (MFMA kernels).
#include "mala_kernels.hpp"

namespace mala {

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
    (void)a; (void)s;
    return hipErrorNotSupported;
}

}  // namespace mala
