// ltxnorm_bf16.hip -- kernel instances for bfloat16 activations, weights and
// outputs (binary32 arithmetic).  The kernels are in ltxnorm_kernels.h and
// ltxnorm_general.h; one translation unit per I/O type keeps builds parallel.
#include "ltxnorm_dispatch.h"

namespace ltxnorm_detail {

ltxnorm_status launch_bf16(Op op, const Request& r, hipStream_t stream) {
    return launch_op<IoBf16>(op, r, stream);
}

}  // namespace ltxnorm_detail
