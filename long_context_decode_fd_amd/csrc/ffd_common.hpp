// Device helpers of the FFD kernels ("Faster Than Flash" digest,
// longzhangge.com, section 5: a 2-bit main part and an 8-bit residual per
// key): the key format's conversions to exact bf16 matrix operands and the
// group-stacked query operand of the matrix-core scan and refine.
#pragma once

#include "internal.hpp"
#include "splitkv.hpp"

namespace fdk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <class T>
__device__ __forceinline__ T ffd_load(const T* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ float half_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// bf16 pair (4 + c[2p], 4 + c[2p+1]) from a code word (dims 2p at bits 2p,
// 2p+1 at bits 16+2p): rotate both 2-bit fields to mantissa bits 5..6 of
// their half and set the exponent of 4.0 (bf16 0x4080 + c*0x20 = 4 + c).
__device__ __forceinline__ uint32_t code_pair(uint32_t w, int p) {
  const uint32_t rot = __builtin_amdgcn_alignbit(w, w, (uint32_t)((2 * p - 5) & 31));
  return (rot & 0x00600060u) | 0x40804080u;
}

// bf16 pair from two small integers held exactly in fp32 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16_exact(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// Query operand of the group-stacked tiles (d = 128): for tile tt (heads
// 4*tt .. 4*tt+3), lane (row i = lane % 16, quad g = lane / 16) at k-step t
// holds q[head 4*tt + i % 4][dims 32g + 8t .. +8] if row i belongs to group
// g (i / 4 == g), zeros otherwise; qsum[tt][e] = sum of q over group g for
// head 4*tt + e.  q points at head 0 of the kv-group.
template <int G>
__device__ __forceinline__ void stacked_query(const uint16_t* q, int lane, u32x4 (&qa)[G / 4][4],
                                              float (&qsum)[G / 4][4]) {
  constexpr int D = 128;
  const int n16 = lane & 15, qg = lane >> 4;
#pragma unroll
  for (int tt = 0; tt < G / 4; ++tt) {
    const uint16_t* qrow = q + (4 * tt + (n16 & 3)) * D + 32 * qg;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      qa[tt][t] = (n16 >> 2) == qg ? ld16(qrow + 8 * t) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t* qh = q + (4 * tt + e) * D + 32 * qg;
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 w = ld16(qh + 8 * t);
        sum += (bf16_lo(w.x) + bf16_hi(w.x)) + (bf16_lo(w.y) + bf16_hi(w.y)) +
               (bf16_lo(w.z) + bf16_hi(w.z)) + (bf16_lo(w.w) + bf16_hi(w.w));
      }
      qsum[tt][e] = sum;
    }
  }
}

__device__ __forceinline__ f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x16(const u32x2& a, const u32x2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                    __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// Four residual bytes (dims in byte order) -> two bf16 pairs of r + 128, exact.
__device__ __forceinline__ u32x2 residual_pairs(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  return u32x2{pack_bf16_exact((float)(u & 0xFF), (float)((u >> 8) & 0xFF)),
               pack_bf16_exact((float)((u >> 16) & 0xFF), (float)(u >> 24))};
}

}  // namespace fdk
