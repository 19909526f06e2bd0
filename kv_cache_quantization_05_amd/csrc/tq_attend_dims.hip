// Explicit instantiations of the general decode-attention launchers of
// tq_attend_v1.h (query kernel, split-K partial kernels for every K/V bit
// width, QJL setting and GQA ratio, merge kernel) for one head dimension per
// object file: the build compiles this source once per d in {32, 64, 128,
// 256} with -DTQ_HEAD_DIM=d, so the four sets of kernels compile in parallel.
#include "tq_attend_v1.h"

#ifndef TQ_HEAD_DIM
#error "compile once per head dimension: -DTQ_HEAD_DIM=32, 64, 128 or 256"
#endif
static_assert(TQ_HEAD_DIM == 32 || TQ_HEAD_DIM == 64 || TQ_HEAD_DIM == 128 || TQ_HEAD_DIM == 256,
              "head dimension 32, 64, 128 or 256");

namespace tq {
namespace v1 {

template hipError_t launch_attend_d<TQ_HEAD_DIM>(const dev_tables &, const dev_tables &, const attend_args &,
                                                 hipStream_t);
template hipError_t launch_prep_d<TQ_HEAD_DIM>(const dev_tables &, const float *, int64_t, float *, int64_t,
                                               hipStream_t);

}  // namespace v1
}  // namespace tq
