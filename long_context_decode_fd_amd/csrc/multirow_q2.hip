// Multi-row decode, two query tiles (16 < G*M <= 32 rows per kv-head).  A
// translation unit of its own so that the build can give it the
// matrix-instruction form that keeps accumulators in ordinary vector
// registers (see build.py): with two tiles that removes most copies between
// the two register files.
#include "multirow.hpp"

namespace fdk {

hipError_t launch_multi_q2(int D, const MultiArgs& a, hipStream_t s) {
  if (D == 64) return launch_multi_d<64, 2>(a, s);
  if (D == 128) return launch_multi_d<128, 2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fdk
