// cg_output.hip -- the CG/output kernels for fp32 q/k/v and for bf16 q/k/v at
// d = 16, and the dispatch by dtype (the bf16 instantiations at d >= 32 are
// in cg_output_bf16.hip).  See cg_output_kernels.h.
#include "cg_output_kernels.h"

namespace mesa {

hipError_t launch_cg_output(const CgOutputArgs& a, hipStream_t s) {
    if (!a.bf16) return dispatch_d<float>(a, s);
    return a.d == 16 ? dispatch_c<16, bf16_t>(a, s) : launch_cg_output_bf16(a, s);
}

}  // namespace mesa
