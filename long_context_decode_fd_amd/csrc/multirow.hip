// Multi-row decode, one query tile (G*M <= 16 rows per kv-head), and the
// dispatch between one and two tiles (the kernel is in multirow.hpp).
#include "multirow.hpp"

namespace fdk {

hipError_t launch_multi_q2(int D, const MultiArgs& a, hipStream_t s);

hipError_t launch_multi(int D, const MultiArgs& a, hipStream_t s) {
  if ((a.Hq / a.Hkv) * a.M > 16) return launch_multi_q2(D, a, s);
  if (D == 64) return launch_multi_d<64, 1>(a, s);
  if (D == 128) return launch_multi_d<128, 1>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fdk
