// Device helpers of the FFD kernels ("Faster Than Flash" digest,
// longzhangge.com, section 5: a 2-bit main part and an 8-bit residual per
// key): the key format's conversions to exact bf16 (dot-product kernel) and
// fp16 (matrix-core kernel) operands, and the group-stacked fp16 query
// operand of the matrix-core scan and refine.
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

// fp16 pair (4 + c[2p], 4 + c[2p+1]) from a code word (dims 2p at bits 2p,
// 2p+1 at bits 16+2p): rotate both 2-bit fields to bits 8..9 of their half
// (the units digit of a half in [4, 8)) and set the exponent of 4.0 (fp16
// 0x4400 + c*0x100 = 4 + c).  mask = 0x03000300 and exp = 0x44004400 come
// in registers: v_and_or_b32 takes no literal.
__device__ __forceinline__ uint32_t code_pair_f16(uint32_t w, int p, uint32_t mask, uint32_t exp) {
  return (__builtin_amdgcn_alignbit(w, w, (uint32_t)((2 * p - 8) & 31)) & mask) | exp;
}

// Four residual bytes r (two's complement, dims in byte order) -> two fp16
// pairs of 1024 + (r + 128): a half in [1024, 2048) has units in its ten
// mantissa bits, so the byte u = r + 128 is the low byte of the half and
// 0x64 its high byte -- one byte permute per pair.  k64 holds 0x64646464.
__device__ __forceinline__ u32x2 residual_pairs_f16(uint32_t w, uint32_t k64) {
  const uint32_t u = w ^ 0x80808080u;
  // perm bytes 0-3 come from the second operand, 4-7 from the first
  return u32x2{__builtin_amdgcn_perm(k64, u, 0x04010400u),
               __builtin_amdgcn_perm(k64, u, 0x04030402u)};
}

// Query operand of the group-stacked tiles (d = 128) as fp16: for tile tt
// (heads 4*tt .. 4*tt+3), lane (row i = lane % 16, quad g = lane / 16) at
// k-step t holds pw * q[head 4*tt + i % 4][dims 32g + 8t .. +8] if row i
// belongs to group g (i / 4 == g), zeros otherwise; qsum[tt][e] = pw * the
// sum of q over group g for head 4*tt + e.  q points at head 0 of the
// kv-group.  Returns pw, the power of two 2^k that brings the largest |q|
// of the G heads into [2^14, 2^15): every scaled element at or above 2^-14
// is then exact in fp16 (11 significant bits against bf16's 8), the smaller
// ones within 2^-25 (the subnormal step), and nothing reaches fp16's 65504.
// Scaling by 2^k commutes with every fp32 rounding of the products and
// sums built on it, so scores from the scaled query are exactly 2^k times
// the unscaled ones.  Two parts: query_load issues one load per element and
// lane (head 4 tt + lane % 4, group lane / 16: the wave covers each element
// four times), stacked_query_f16 builds the operand from them, so that other
// loads can be issued in between.  Wave-uniform result.
template <int G>
__device__ __forceinline__ void query_load(const uint16_t* q, int lane, u32x4 (&raw)[G / 4][4]) {
  constexpr int D = 128;
  const int n16 = lane & 15, qg = lane >> 4;
#pragma unroll
  for (int tt = 0; tt < G / 4; ++tt)
#pragma unroll
    for (int t = 0; t < 4; ++t) raw[tt][t] = ld16(q + (4 * tt + (n16 & 3)) * D + 32 * qg + 8 * t);
}
template <int G>
__device__ __forceinline__ float stacked_query_f16(const u32x4 (&raw)[G / 4][4], int lane,
                                                   u32x4 (&qa)[G / 4][4],
                                                   float (&qsum)[G / 4][4]) {
  constexpr int NT = G / 4;
  const int n16 = lane & 15, qg = lane >> 4;
  float mx = 0.f, own[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 w = raw[tt][t];
      sum += (bf16_lo(w.x) + bf16_hi(w.x)) + (bf16_lo(w.y) + bf16_hi(w.y)) +
             (bf16_lo(w.z) + bf16_hi(w.z)) + (bf16_lo(w.w) + bf16_hi(w.w));
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(bf16_lo(w.x)), fabsf(bf16_hi(w.x))),
                           fmaxf(fabsf(bf16_lo(w.y)), fabsf(bf16_hi(w.y)))));
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(bf16_lo(w.z)), fabsf(bf16_hi(w.z))),
                           fmaxf(fabsf(bf16_lo(w.w)), fabsf(bf16_hi(w.w)))));
    }
    own[tt] = sum;   // head 4 tt + n16 % 4, group qg
  }
  mx = wave_max(mx);
  float pw = 1.f;    // zero, inf or NaN query: unscaled
  if (mx > 0.f && mx != __builtin_inff()) {
    int e = 0;
    (void)frexpf(mx, &e);   // mx in [2^(e-1), 2^e)
    pw = ldexpf(1.f, min(max(15 - e, -126), 126));
  }
  auto half2 = [&](uint32_t w) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_pkrtz(bf16_lo(w) * pw, bf16_hi(w) * pw));
  };
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) qsum[tt][e] = __shfl(own[tt], 16 * qg + e) * pw;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 w = raw[tt][t];
      qa[tt][t] = (n16 >> 2) == qg ? u32x4{half2(w.x), half2(w.y), half2(w.z), half2(w.w)}
                                   : u32x4{0, 0, 0, 0};
    }
  }
  return pw;
}

__device__ __forceinline__ f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_16x16x32_f16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                 __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

}  // namespace fdk
