// Building blocks of one split-KV unit, shared by the dense/paged/fixed-max
// kernel and the FFD kernel.
//
// Lane layout ("row slots"): a cache row of D elements is read by kLpt lanes
// with 16 bytes each; a wave load covers kTpl consecutive rows.  Lane
// (grp = lane / kLpt, col = lane % kLpt) owns dims [col*kVec, col*kVec + kVec)
// of row slot grp.  Every row slot keeps its own softmax state (m, l, O) for
// the G query heads of the kv-head; slots are merged once at the end of the
// unit ("Flash Decoding" explainer, section 2: the same exact merge that
// joins chunks joins slots).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace fdk {

constexpr int kWaves = 4;      // wavefronts per workgroup
constexpr int kThreads = kWaves * kWave;
// Load instructions per tensor per wave in one batch of the split-KV
// kernels (the K and V loads of a batch): deep batches keep many 16-byte
// loads in flight per wave, but the K, V and score registers of a batch grow
// with the depth and with G (8 measured 7 % slower than 16, 20 no better).
constexpr int kBatchLoads = 16;
template <int G>
constexpr int batch_rows() { return G >= 8 ? 8 : kBatchLoads; }

// Lane layout of a cache row: each of kLpt lanes holds P 16-byte pieces of
// the row; piece p of lane `col` is bytes [p * kRow / P + col * 16, +16).
// One wave load instruction (fixed p) covers kTpl rows.  More pieces per
// lane mean fewer lanes per row, hence fewer butterfly steps per score and
// fewer lanes that redo the per-row exponential.
template <typename E, int D, int P = 1>
struct Geo {
  static constexpr int kPieces = P;
  static constexpr int kPv = 16 / (int)sizeof(E);    // elements per piece
  static constexpr int kVec = P * kPv;               // elements per lane per row
  static constexpr int kLpt = D / kVec;              // lanes per cache row
  static constexpr int kTpl = kWave / kLpt;          // rows per wave load
  static constexpr int kRow = D * (int)sizeof(E);    // bytes per cache row
  static_assert(kLpt == 4 || kLpt == 8 || kLpt == 16 || kLpt == 32, "row split");
  // element index (0..D) of a lane's value e
  static __device__ __forceinline__ int dim(int col, int e) {
    return (e / kPv) * (D / P) + col * kPv + e % kPv;
  }
};

// q . k over one lane's 16-byte slice.
template <typename E>
__device__ __forceinline__ float slice_dot(const u32x4& q, const u32x4& k) {
  if constexpr (std::is_same<E, uint16_t>::value) {
    // one accumulation chain: v_dot2c accumulates into its destination, so
    // every extra chain costs a zero-initialising move
    float a = dot2_bf16(q.x, k.x, 0.f);
    a = dot2_bf16(q.y, k.y, a);
    a = dot2_bf16(q.z, k.z, a);
    return dot2_bf16(q.w, k.w, a);
  } else {
    float a = __uint_as_float(q.x) * __uint_as_float(k.x);
    float b = __uint_as_float(q.y) * __uint_as_float(k.y);
    a = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), a);
    b = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), b);
    return a + b;
  }
}

// q . k over a lane's P pieces, one accumulation chain.
template <typename E, int P>
__device__ __forceinline__ float pieces_dot(const u32x4* q, const u32x4* k) {
  if constexpr (std::is_same<E, uint16_t>::value) {
    float a = dot2_bf16(q[0].x, k[0].x, 0.f);
    a = dot2_bf16(q[0].y, k[0].y, a);
    a = dot2_bf16(q[0].z, k[0].z, a);
    a = dot2_bf16(q[0].w, k[0].w, a);
#pragma unroll
    for (int p = 1; p < P; ++p) {
      a = dot2_bf16(q[p].x, k[p].x, a);
      a = dot2_bf16(q[p].y, k[p].y, a);
      a = dot2_bf16(q[p].z, k[p].z, a);
      a = dot2_bf16(q[p].w, k[p].w, a);
    }
    return a;
  } else {
    float a = slice_dot<E>(q[0], k[0]);
#pragma unroll
    for (int p = 1; p < P; ++p) a += slice_dot<E>(q[p], k[p]);
    return a;
  }
}

// One lane's 16-byte slice of a V row as fp32.
template <typename E>
__device__ __forceinline__ void slice_vals(const u32x4& v, float* f) {
  if constexpr (std::is_same<E, uint16_t>::value) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

template <int G, int VEC>
__device__ __forceinline__ void state_reset(float (&acc)[G][VEC], float (&m)[G],
                                            float (&l)[G]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
  }
}

// Exponentials of one cache row for the G heads of the kv-head:
// p[h] = exp2(f(x[h], y[h])).  Every lane of a row holds the same x and y
// (the row sums are reduced symmetrically), so for G = 2 or 4 each lane
// evaluates only head lane % G and takes the others from the lanes of its
// quad, which hold heads 0 .. G-1 of the same row: one exponential (a
// quarter-rate instruction) and G moves instead of G exponentials, with the
// same bits.  F maps (x, y) to the exponent.
template <int G, class F>
__device__ __forceinline__ void row_exp2(const float (&x)[G], const float (&y)[G], F f,
                                         float (&p)[G]) {
  if constexpr (G == 2 || G == 4) {
    const int hs = (int)(threadIdx.x % G);
    float xs = x[0], ys = y[0];
#pragma unroll
    for (int h = 1; h < G; ++h) {
      xs = hs == h ? x[h] : xs;
      ys = hs == h ? y[h] : ys;
    }
    const float pm = exp2_hw(f(xs, ys));
    p[0] = dpp<0x00>(pm);   // quad_perm [0,0,0,0]
    p[1] = dpp<0x55>(pm);   // quad_perm [1,1,1,1]
    if constexpr (G == 4) {
      p[2] = dpp<0xAA>(pm);
      p[3] = dpp<0xFF>(pm);
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) p[h] = exp2_hw(f(x[h], y[h]));
  }
}

// Online-softmax update of a row slot with a batch of NB rows.
// s[i][h]: raw dot products q_h . k_i (-inf for rows that do not count);
// m[h]: running maximum in the same raw units.  The accumulator is rescaled
// only when some slot of the wave saw a larger maximum.
template <typename E, int G, int VEC, int NB, int P = 1>
__device__ __forceinline__ void online_update(const float (&s)[NB][G],
                                              const u32x4 (&vr)[NB * P], float c_log2,
                                              float (&acc)[G][VEC], float (&m)[G],
                                              float (&l)[G]) {
  float mb[G];
  bool grow = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mb[h] = m[h];
#pragma unroll
    for (int i = 0; i < NB; ++i) mb[h] = fmaxf(mb[h], s[i][h]);
    grow |= mb[h] > m[h];
  }
  if (__any(grow)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = (mb[h] == m[h]) ? 1.f : exp2_hw((m[h] - mb[h]) * c_log2);
      l[h] *= a;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] *= a;
      m[h] = mb[h];
    }
  }
  // exponent (s - m) * c: exactly 0, so p exactly 1, at the row that holds
  // the running maximum (a single key returns its value bit for bit)
  float base[G];
#pragma unroll
  for (int h = 0; h < G; ++h) base[h] = (m[h] == kNegInf) ? 0.f : m[h];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float vf[VEC];
#pragma unroll
    for (int pc = 0; pc < P; ++pc) slice_vals<E>(vr[i * P + pc], vf + pc * (VEC / P));
    float p[G];
    row_exp2<G>(s[i], base, [c_log2](float x, float b) { return (x - b) * c_log2; }, p);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] += p[h];
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(p[h], vf[e], acc[h][e]);
    }
  }
}

// Raw running maximum -> log2 units of the scaled score.
template <int G>
__device__ __forceinline__ void state_to_log2(float (&m)[G], float c_log2) {
#pragma unroll
  for (int h = 0; h < G; ++h) m[h] = (m[h] == kNegInf) ? kNegInf : m[h] * c_log2;
}

// One exchange of the slot merge: lanes i and i ^ OFF combine their states
// (then OFF * 2, ... up to 32).  Both lanes of a pair compute the same
// symmetric expression, so they end with identical bits; the two weighted
// terms are rounded separately before the add (no fused multiply-add).
template <int OFF, int G, int VEC>
__device__ __forceinline__ void slot_merge_step(float (&acc)[G][VEC], float (&m)[G],
                                                float (&l)[G]) {
#pragma clang fp contract(off)
  if constexpr (OFF < kWave) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float ma, mb, la, lb;
      lane_pair<OFF>(m[h], ma, mb);
      lane_pair<OFF>(l[h], la, lb);
      const float M = fmaxf(ma, mb);
      const float wa = exp2_diff(ma, M), wb = exp2_diff(mb, M);
      l[h] = la * wa + lb * wb;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float xa, xb;
        lane_pair<OFF>(acc[h][e], xa, xb);
        acc[h][e] = xa * wa + xb * wb;
      }
      m[h] = M;
    }
    slot_merge_step<OFF * 2, G, VEC>(acc, m, l);
  }
}

// Reduce-scatter of the row slots' states at a unit's end (the same exact
// merge as slot_merge_step, split so that no lane does all of it).  First the
// largest slot maximum M per head and one rescale of each slot to it
// (2^(m - M)); the exchanges then only add.  Exchanges over fewer than 16
// lanes (DPP) add every value; the exchanges over 16 and 32 lanes swap two
// different values per instruction (v_permlane16_swap / v_permlane32_swap
// of x_k with x_{k + n/2}): lanes of one half receive both lanes' x_k, the
// others both lanes' x_{k + n/2}, so each lane adds and keeps half, then a
// quarter, of the values.  Each step adds two values (commutative), so the
// result does not depend on which lane computes it.  Afterwards m = M
// and l (summed over all slots) are the same in every lane, and kept[k] is
// the merged value of flat index h * VEC + e = index(lane, k).
template <int LPT, int G, int VEC>
struct SlotScatter {
  static constexpr int NV = G * VEC;
  // the exchange over 32 lanes always splits; the one over 16 lanes splits
  // too when it starts below 32 lanes and leaves at least 4 values per lane
  // (16-byte stores), otherwise it adds every value
  static constexpr bool S16 = LPT <= 16 && NV >= 16;
  static constexpr int NK = NV >> (S16 ? 2 : 1);   // values each lane keeps
  static __device__ __forceinline__ int index(int lane, int k) {
    if constexpr (S16)
      return ((lane >> 4) & 1) * (NV / 2) + ((lane >> 5) & 1) * (NV / 4) + k;
    else
      return ((lane >> 5) & 1) * (NV / 2) + k;
  }
  // Lanes that differ only in the bits of the adding exchanges (DUP) hold
  // the same values: NCOPY copies of each, told apart by copy(lane).
  static constexpr int DUP = (LPT < 16 ? 16 - LPT : 0) | (!S16 && LPT <= 16 ? 16 : 0);
  static constexpr int NCOPY = 64 * NK / (LPT * NV);
  static __device__ __forceinline__ int copy(int lane) {
    int r = 0, o = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      if ((DUP >> bit) & 1) {
        r |= ((lane >> bit) & 1) << o;
        ++o;
      }
    }
    return r;
  }
};

template <int OFF>
__device__ __forceinline__ float slot_max(float x) {
  if constexpr (OFF < kWave) return slot_max<OFF * 2>(pair_max<OFF>(x));
  else return x;
}
template <int OFF>
__device__ __forceinline__ float slot_sum(float x) {
  if constexpr (OFF < kWave) return slot_sum<OFF * 2>(pair_sum<OFF>(x));
  else return x;
}

__device__ __forceinline__ void swap_add16(float x, float y, float& out) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                  false);
  out = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap_add32(float x, float y, float& out) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                  false);
  out = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int LPT, int G, int VEC>
__device__ __forceinline__ void slot_reduce_scatter(
    float (&acc)[G][VEC], float (&m)[G], float (&l)[G],
    float (&kept)[(G * VEC) >> ((LPT <= 16 && G * VEC >= 16) ? 2 : 1)]) {
  using SS = SlotScatter<LPT, G, VEC>;
  constexpr int NV = SS::NV;
  float x[NV];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = slot_max<LPT>(m[h]);
    const float f = exp2_diff(m[h], M);
    l[h] = slot_sum<LPT>(l[h] * f);
    m[h] = M;
#pragma unroll
    for (int e = 0; e < VEC; ++e) x[h * VEC + e] = acc[h][e] * f;
  }
  // DPP exchanges (offsets LPT .. 8): full sums
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if constexpr (LPT <= 4) x[k] = pair_sum<4>(x[k]);
    if constexpr (LPT <= 8) x[k] = pair_sum<8>(x[k]);
  }
  if constexpr (SS::S16) {
    float y[NV / 2];
#pragma unroll
    for (int k = 0; k < NV / 2; ++k) swap_add16(x[k], x[k + NV / 2], y[k]);
#pragma unroll
    for (int k = 0; k < NV / 4; ++k) swap_add32(y[k], y[k + NV / 4], kept[k]);
  } else {
    if constexpr (LPT <= 16) {
#pragma unroll
      for (int k = 0; k < NV; ++k) x[k] = pair_sum<16>(x[k]);
    }
#pragma unroll
    for (int k = 0; k < NV / 2; ++k) swap_add32(x[k], x[k + NV / 2], kept[k]);
  }
}

// LDS scratch of the unit combine.
template <int G, int D>
struct CombineLds {
  float acc[kWaves][G][D];
  float ml[kWaves][G][2];
};

// Merge the row slots of every wave, then the waves, and write the unit's
// partial for each of its G query heads: O (unnormalised, relative to m),
// m (log2 units) and l.  m must already be in log2 units.  `prow0` is the
// partial row index of query head 0 of the group; heads are `hstride` rows
// apart.
template <int G, int D, int VEC, int LPT>
__device__ __forceinline__ void combine_store(CombineLds<G, D>& lds, float (&acc)[G][VEC],
                                              float (&m)[G], float (&l)[G], float* o_part,
                                              float* ml_part, size_t prow0, size_t hstride) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
  slot_merge_step<LPT, G, VEC>(acc, m, l);
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; e += 4)
        *reinterpret_cast<f32x4*>(&lds.acc[wave][h][lane * VEC + e]) =
            f32x4{acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]};
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lds.ml[wave][h][0] = m[h];
      lds.ml[wave][h][1] = l[h];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D, dd = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds.ml[w][h][0]);
    float o = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = exp2_diff(lds.ml[w][h][0], M);
      o = fmaf(wt, lds.acc[w][h][dd], o);
      ls = fmaf(wt, lds.ml[w][h][1], ls);
    }
    const size_t prow = prow0 + (size_t)h * hstride;
    o_part[prow * D + dd] = o;
    if (dd == 0) {
      ml_part[prow * 2] = M;
      ml_part[prow * 2 + 1] = ls;
    }
  }
}

}  // namespace fdk
