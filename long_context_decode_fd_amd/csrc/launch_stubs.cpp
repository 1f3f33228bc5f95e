// Kernel-launch stand-ins for the host-sanitizer build only (see build.py,
// build_sanitized_host): the C ABI's validation, workspace sizing and error
// paths (api.hip) are compiled with AddressSanitizer and UndefinedBehavior-
// Sanitizer and run on a machine without a GPU.  Those checks never reach a
// launch; if one did, it stops here instead of touching a device.
#include <stdio.h>
#include <stdlib.h>

#include "internal.hpp"

namespace fdk {

[[noreturn]] static void no_launch(const char* what) {
  fprintf(stderr, "host-sanitizer build: the %s launch was reached\n", what);
  abort();
}

hipError_t launch_partial(int, int, int, int, const PartialArgs&, hipStream_t) {
  no_launch("partial kernel");
}
hipError_t launch_merge(int, int, const MergeArgs&, hipStream_t) { no_launch("merge kernel"); }
hipError_t launch_range_flags(const float*, uint8_t*, size_t, float, float, hipStream_t) {
  no_launch("range flags kernel");
}
hipError_t launch_ffd_pack(int, const FfdPackArgs&, hipStream_t) { no_launch("FFD pack kernel"); }
hipError_t launch_ffd(int, int, const FfdArgs&, hipStream_t) { no_launch("FFD kernel"); }
hipError_t launch_multi(int, const MultiArgs&, hipStream_t) { no_launch("multi-row kernel"); }
int multi_fold(int, const MultiArgs&) { no_launch("multi-row split"); }
hipError_t launch_append(bool, const AppendArgs&, hipStream_t) { no_launch("append kernel"); }

}  // namespace fdk
