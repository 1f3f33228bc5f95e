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

// Scan B operand of one k-step from a code word (dims 2p at bits 2p, 2p+1
// at bits 16+2p; k-step parity h takes pairs 4h .. 4h+3): after a right
// shift by 8h, pair i of the k-step sits at bits 2i and 16+2i, and the mask
// leaves each half the fp16 subnormal c 2^(2i-24) (mantissa bits 2i, 2i+1):
// exact, and with no offset to cancel later.  The matching query operand
// carries pw 2^-2i (stacked_query_f16), so each product is 2^-24 pw q c,
// exact in fp32.
__device__ __forceinline__ u32x4 code_operand_f16(uint32_t w, int h) {
  const uint32_t x = h ? w >> 8 : w;
  return u32x4{x & 0x00030003u, x & 0x000C000Cu, x & 0x00300030u, x & 0x00C000C0u};
}

// Four residual bytes r (two's complement, dims in byte order) -> two fp16
// pairs of the subnormals u 2^-24, u = r + 128: the byte u is the mantissa
// of a half whose other bits are zero -- one byte permute per pair
// (selector 12 gives a zero byte; bytes 0-3 come from the second operand).
__device__ __forceinline__ u32x2 residual_pairs_f16(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  return u32x2{__builtin_amdgcn_perm(u, u, 0x0C010C00u), __builtin_amdgcn_perm(u, u, 0x0C030C02u)};
}

// Query operands of the group-stacked tiles (d = 128) as fp16: for tile tt
// (heads 4*tt .. 4*tt+3), lane (row i = lane % 16, quad g = lane / 16) at
// k-step t holds pw * q[head 4*tt + i % 4][dims 32g + 8t .. +8] if row i
// belongs to group g (i / 4 == g), zeros otherwise (qa, the refine's
// operand); qs, the scan's, holds the same values times 2^-2j for the pair
// j = 0 .. 3 of each 32-bit word (the code operand's halves are c 2^(2j-24),
// so each product is 2^-24 pw q c); qsum[tt][e] = pw * the sum of q over
// group g for head 4*tt + e.  q points at head 0 of the kv-group.  Returns
// pw, the power of two 2^k that brings the largest |q| of the G heads into
// [2^14, 2^15): every scaled element at or above 2^-14 is then exact in
// fp16 (11 significant bits against bf16's 8), the smaller ones within
// 2^-25 (qa) and 2^-19 (qs, after its 2^-2j) of pw q, and nothing reaches
// fp16's 65504.  Scaling by powers of two commutes with every fp32 rounding
// of the products and sums built on them, so scores from the scaled query
// are exactly 2^k (scan: 2^(k-24)) times the unscaled ones.  Two parts:
// query_load issues one load per element and lane (head 4 tt + lane % 4,
// group lane / 16: the wave covers each element four times),
// stacked_query_f16 builds the operands from them, so that other loads can
// be issued in between.  Wave-uniform result.
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
                                                   u32x4 (&qs)[G / 4][4],
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
  auto half2 = [&](uint32_t w, float f) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_pkrtz(bf16_lo(w) * f, bf16_hi(w) * f));
  };
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) qsum[tt][e] = __shfl(own[tt], 16 * qg + e) * pw;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 w = raw[tt][t];
      const bool own_group = (n16 >> 2) == qg;
      qa[tt][t] = own_group ? u32x4{half2(w.x, pw), half2(w.y, pw), half2(w.z, pw), half2(w.w, pw)}
                            : u32x4{0, 0, 0, 0};
      qs[tt][t] = own_group ? u32x4{half2(w.x, pw), half2(w.y, pw * 0x1p-2f),
                                    half2(w.z, pw * 0x1p-4f), half2(w.w, pw * 0x1p-6f)}
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
