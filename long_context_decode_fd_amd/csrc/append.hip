// Cache append for gfx950: the decode step's new key/value rows written into
// a contiguous cache or a paged pool ("Flash Decoding" explainer, section 3:
// every generated token appends its K and V to the cache, which a paged
// cache keeps in fixed-size pages found through the block table).
//
// One thread per 16 bytes of new rows; K and V together.  Paged positions
// come from the device (one write position per sequence), and a position
// whose page is outside the table, or whose table entry is not a valid page,
// is skipped rather than written.
#include "internal.hpp"

#include "common.hpp"

namespace fdk {

constexpr int kAppendThreads = 256;

template <bool PAGED>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int per_row = a.row_bytes / 16;
  const size_t total = (size_t)a.B * a.Hkv * a.M * per_row;
  const size_t stride = (size_t)gridDim.x * kAppendThreads;
  for (size_t i = (size_t)blockIdx.x * kAppendThreads + threadIdx.x; i < total; i += stride) {
    const int c = (int)(i % per_row);
    size_t r = i / per_row;
    const int m = (int)(r % a.M);
    r /= a.M;
    const int kvh = (int)(r % a.Hkv);
    const int b = (int)(r / a.Hkv);
    size_t dst_row;
    if constexpr (PAGED) {
      const int p = a.pos[b] + m;
      if (p < 0) continue;
      const int pi = p >> a.page_shift;
      if (pi >= a.max_pages) continue;
      const int page = a.block_table[(size_t)b * a.max_pages + pi];
      if (page < 0 || page >= a.num_pages) continue;
      dst_row = (((size_t)page * a.Hkv + kvh) << a.page_shift) |
                (size_t)(p & ((1 << a.page_shift) - 1));
    } else {
      dst_row = ((size_t)b * a.Hkv + kvh) * (size_t)a.L_cap + (size_t)(a.t0 + m);
    }
    const size_t src = (((size_t)b * a.Hkv + kvh) * a.M + m) * (size_t)a.row_bytes + (size_t)c * 16;
    const size_t dst = dst_row * (size_t)a.row_bytes + (size_t)c * 16;
    *reinterpret_cast<u32x4*>(a.k_dst + dst) = *reinterpret_cast<const u32x4*>(a.k_new + src);
    *reinterpret_cast<u32x4*>(a.v_dst + dst) = *reinterpret_cast<const u32x4*>(a.v_new + src);
  }
}

hipError_t launch_append(bool paged, const AppendArgs& a, hipStream_t s) {
  const size_t total = (size_t)a.B * a.Hkv * a.M * (a.row_bytes / 16);
  const size_t blocks = (total + kAppendThreads - 1) / kAppendThreads;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536)), block(kAppendThreads);
  if (paged) hipLaunchKernelGGL((append_kernel<true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((append_kernel<false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace fdk
