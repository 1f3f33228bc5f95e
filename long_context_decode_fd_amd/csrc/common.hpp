// Device helpers shared by the decode-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdk {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// exp2(a - b) that is 0 (not NaN) when both are -inf.
__device__ __forceinline__ float exp2_diff(float a, float b) {
  return exp2_hw(a - (b == kNegInf ? 0.f : b));
}

// Lane permutation inside a row of 16 lanes (DPP); every source lane is valid
// for the controls used here, so no bound control is needed.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

enum : int {
  kQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]
  kQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]
  kRowHalfMirror = 0x141, // lane i <-> 7-i inside each half row
  kRowMirror = 0x140,     // lane i <-> 15-i inside each row
};

// The two values of lane i's pair {i, i ^ OFF} (OFF = 4, 8, 16 or 32),
// without the LDS crossbar: a and b are the pair's two values (for OFF >= 16
// in the order lower lane, upper lane in both lanes; for OFF < 16 own value,
// then the partner's).  Results that are symmetric in a and b are therefore
// bitwise equal in both lanes.  Every lane of the wave must be active.
template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  static_assert(OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32, "pair offset");
  if constexpr (OFF == 16 || OFF == 32) {
    // v_permlane{16,32}_swap of x with itself: element 0 holds lane
    // i & ~OFF's value, element 1 lane i | OFF's
    const uint32_t u = __float_as_uint(x);
    const auto r = OFF == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else if constexpr (OFF == 8) {
    a = x;
    b = dpp<0x128>(x);   // row_ror:8 = lane i ^ 8 inside a row of 16
  } else {
    const float up = dpp<0x104>(x);   // row_shl:4: lane i + 4
    const float dn = dpp<0x114>(x);   // row_shr:4: lane i - 4
    a = x;
    b = (__lane_id() & 4) ? dn : up;
  }
}

// Sum and maximum over lane i's pair {i, i ^ OFF}, the same bits in both lanes.
template <int OFF>
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  lane_pair<OFF>(x, a, b);
  return a + b;
}
template <int OFF>
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  lane_pair<OFF>(x, a, b);
  return fmaxf(a, b);
}

// Sum over aligned groups of N lanes (N = 4, 8, 16 or 32); every lane of the
// group receives the group's sum.  After the two quad steps each quad holds
// its sum; the half-row mirror pairs lane i with a lane of the other quad,
// the row mirror pairs the two halves, and a pair exchange joins two rows of 16.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kRowMirror>(x);
  if constexpr (N >= 32) x = pair_sum<16>(x);
  return x;
}

// group_sum over every element of an array, one butterfly step at a time
// across the whole array, so no step waits on the one just issued.
template <int N, int M>
__device__ __forceinline__ void group_sum_n(float (&x)[M]) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
#pragma unroll
  for (int k = 0; k < M; ++k) x[k] += dpp<kQuadXor1>(x[k]);
#pragma unroll
  for (int k = 0; k < M; ++k) x[k] += dpp<kQuadXor2>(x[k]);
  if constexpr (N >= 8) {
#pragma unroll
    for (int k = 0; k < M; ++k) x[k] += dpp<kRowHalfMirror>(x[k]);
  }
  if constexpr (N >= 16) {
#pragma unroll
    for (int k = 0; k < M; ++k) x[k] += dpp<kRowMirror>(x[k]);
  }
  if constexpr (N >= 32) {
#pragma unroll
    for (int k = 0; k < M; ++k) x[k] = pair_sum<16>(x[k]);
  }
}

// Same groups, maximum.
template <int N>
__device__ __forceinline__ float group_max(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kRowHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kRowMirror>(x));
  if constexpr (N >= 32) x = pair_max<16>(x);
  return x;
}

// Whole-wave reductions (used outside the hot loops).
// Pairs at distance 32, 16, 8, 4, 2, 1 in that order, every exchange
// without the LDS crossbar; each step is commutative, so every lane ends with
// the same bits.
__device__ __forceinline__ float wave_max(float x) {
  x = pair_max<4>(pair_max<8>(pair_max<16>(pair_max<32>(x))));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  return fmaxf(x, dpp<kQuadXor1>(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = pair_sum<4>(pair_sum<8>(pair_sum<16>(pair_sum<32>(x))));
  x += dpp<kQuadXor2>(x);
  return x + dpp<kQuadXor1>(x);
}

// bf16 pairs packed in a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 16-byte global loads.  The streaming variant marks them non-temporal: the
// cache is read once per call, and keeping it out of the caches raises the
// sustained read rate on gfx950 (measured ~7.1 vs ~6.3 TB/s for a plain
// streaming read).
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Raw buffer descriptors (gfx9 family): word 3 of a plain byte-addressed
// buffer, and the cache-policy bit that marks a buffer load non-temporal.
constexpr int kBufferDword3 = 0x00020000;
constexpr int kBufferNonTemporal = 2;

// Descriptor of `bytes` bytes at p.  p and bytes must be wave-uniform; they
// are read from the first active lane, so the descriptor lives in scalar
// registers and the loads need no per-lane descriptor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, 0, __builtin_amdgcn_readfirstlane(bytes),
                                           kBufferDword3);
}

// 16-byte non-temporal buffer load at byte offset `off` of descriptor r
// (zeros, and no memory access, when off + 16 exceeds its limit).
__device__ __forceinline__ u32x4 ld16_buf(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufferNonTemporal));
}

}  // namespace fdk
