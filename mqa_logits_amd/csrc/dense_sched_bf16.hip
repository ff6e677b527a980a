// Dense and compressed weighted MQA logits for gfx950: bf16-logits instances
// that follow a work schedule from mqa_logits_metadata.
#include "dense_kernel.hpp"

namespace mqa {

hipError_t launch_dense_sched_bf16(int fmt, int h, int d, int store, const DenseParams& p,
                                   hipStream_t s) {
  return dispatch_fmt<kBF16, true>(fmt, h, d, store, p.exact != 0, p, s);
}

}  // namespace mqa
