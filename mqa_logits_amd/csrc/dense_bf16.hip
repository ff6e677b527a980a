// Dense and compressed weighted MQA logits for gfx950: bf16-logits instances
// split by row chunks (each instance group has a translation unit of its own
// so they compile in parallel).
#include "dense_kernel.hpp"

namespace mqa {

hipError_t launch_dense_bf16(int fmt, int h, int d, int store, const DenseParams& p,
                             hipStream_t s) {
  return dispatch_fmt<kBF16, false>(fmt, h, d, store, p.exact != 0, p, s);
}

}  // namespace mqa
