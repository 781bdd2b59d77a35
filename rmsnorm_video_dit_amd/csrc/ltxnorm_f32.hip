// ltxnorm_f32.hip -- kernel instances for IEEE binary32 activations, weights and
// outputs (binary32 arithmetic).  The kernels are in ltxnorm_kernels.h and
// ltxnorm_general.h; one translation unit per I/O type keeps builds parallel.
#include "ltxnorm_dispatch.h"

namespace ltxnorm_detail {

ltxnorm_status launch_f32(Op op, const Request& r, hipStream_t stream) {
    return launch_op<IoF32>(op, r, stream);
}

}  // namespace ltxnorm_detail
