// Instantiation of the general decode-attention kernels for head_dim 256.
#include "tq_attend_v1.h"

namespace tq {

hipError_t launch_attend_dim256(const dev_tables & kt, const dev_tables & vt, const attend_args & a,
                               hipStream_t s) {
    return v1::launch_attend_d<256>(kt, vt, a, s);
}

hipError_t launch_prep_dim256(const dev_tables & t, const float * q, int64_t n, float * qp, int64_t stride,
                             hipStream_t s) {
    return v1::launch_prep_d<256>(t, q, n, qp, stride, s);
}

}  // namespace tq
