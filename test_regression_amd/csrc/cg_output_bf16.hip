// cg_output_bf16.hip -- the CG/output kernels for bf16 q/k/v at d >= 32 (see
// cg_output_kernels.h); a unit of its own so that the two dtypes' kernels
// compile in parallel.
#include "cg_output_kernels.h"

namespace mesa {

hipError_t launch_cg_output_bf16(const CgOutputArgs& a, hipStream_t s) {
    switch (a.d) {
        case 32: return dispatch_c<32, bf16_t>(a, s);
        case 64: return dispatch_c<64, bf16_t>(a, s);
        case 128: return dispatch_c<128, bf16_t>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mesa
