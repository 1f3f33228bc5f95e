// FFD sparse decode for gfx950 ("Faster Than Flash" digest, longzhangge.com):
// a 2-bit key scan of every position, a pseudo-maximum from attention-sink
// and local-window anchors, top-delta selection, an 8-bit residual refine of
// the candidates and exact attention over them (sections 3-6, Fig. 2), plus
// the packer that produces the key format (section 5).
//
// One workgroup = one unit = (sequence, kv-head, chunk), fused:
//   0. Anchors.  A small kernel scores the anchor positions of every
//      (sequence, kv-head) with the refined key (2-bit + residual) once and
//      leaves m^ and j* per query head in the workspace.
//   1. Scan.  4 lanes per position (one 32-dim quantisation group each) read
//      8 B of codes and 4 B of (zero, step).  Codes become exact bf16 values
//      4 + c (a rotate and an and-or per pair, since bf16 4..7 differ only in
//      two mantissa bits); sum q_i c_i = sum q_i (4 + c_i) - 4 sum q_i.  At
//      d = 128 with G = 4 or 8 the products run on the matrix cores (the
//      groups of 4 heads stacked block-diagonally in one 16x16x32 tile), else
//      in v_dot2c_f32_bf16.  The scan score and the G-bit candidate mask of
//      every position stay in LDS (no write-back).
//   2. Compaction of the positions that are a candidate for any head of the
//      group (they share the residual and V loads).
//   3. Refine + attend over the compacted list: residual bytes become exact
//      bf16 (r + 128); each head's softmax covers only its own candidates.
//      At d = 128 with G = 4 or 8 on the matrix cores, 16 candidates per
//      tile (refinement in the scan's group-stacked tile, P V with the
//      candidates' V rows read back transposed from LDS); else 16 lanes per
//      row with dot2 and V rows streamed as in the dense kernel.
//   4. Row slots and waves merge into one partial per query head; the
//      chunks merge in the common log-sum-exp kernel.
#include <type_traits>

#include "internal.hpp"
#include "splitkv.hpp"

namespace fdk {

// load rounds of the scan (positions per lane per round) and rows per slot
// per batch of the dot-product refine
constexpr int kScanSteps = 8;
constexpr int kScanTiles = 8;   // 16-position tiles per round on the matrix cores
constexpr int kRefineRows = 8;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Dynamic LDS of the FFD kernel for a chunk of `chunk` positions: scan
// scores [chunk][G] (fp32), candidate masks [chunk] (u8), candidate list
// [chunk] (u16).  Sized to the chunk so that short chunks leave room for
// more resident workgroups.
template <int G>
__host__ __device__ constexpr size_t ffd_lds_mask_off(int chunk) { return (size_t)chunk * G * 4; }
template <int G>
__host__ __device__ constexpr size_t ffd_lds_list_off(int chunk) {
  return (ffd_lds_mask_off<G>(chunk) + (size_t)chunk + 3) & ~(size_t)3;
}
template <int G>
__host__ __device__ constexpr size_t ffd_lds_bytes(int chunk) {
  return ffd_lds_list_off<G>(chunk) + (size_t)chunk * 2;
}

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

// Residual part of the refined dot product for one lane's 8 dims:
// rs * sum_i q_i r_i, with the residual bytes read as r + 128 (exact bf16).
template <int G>
__device__ __forceinline__ void residual_dot(const u32x2& rr, float rsf, const u32x4 (&qr)[G],
                                             const float (&ql)[G], float (&out)[G]) {
  const uint32_t u0 = rr.x ^ 0x80808080u, u1 = rr.y ^ 0x80808080u;
  const uint32_t p0 = pack_bf16_exact((float)(u0 & 0xFF), (float)((u0 >> 8) & 0xFF));
  const uint32_t p1 = pack_bf16_exact((float)((u0 >> 16) & 0xFF), (float)(u0 >> 24));
  const uint32_t p2 = pack_bf16_exact((float)(u1 & 0xFF), (float)((u1 >> 8) & 0xFF));
  const uint32_t p3 = pack_bf16_exact((float)((u1 >> 16) & 0xFF), (float)(u1 >> 24));
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float a = dot2_bf16(qr[h].x, p0, 0.f);
    float b = dot2_bf16(qr[h].y, p1, 0.f);
    a = dot2_bf16(qr[h].z, p2, a);
    b = dot2_bf16(qr[h].w, p3, b);
    out[h] = rsf * fmaf(-128.f, ql[h], a + b);
  }
}

// Query slices of the 16-lane (row) layout (dims off .. off + 8 of each head
// of the kv-group) and their sums.
template <int G>
__device__ __forceinline__ void query_sums(const u32x4 (&qr)[G], float (&ql)[G]) {
#pragma unroll
  for (int h = 0; h < G; ++h)
    ql[h] = ((bf16_lo(qr[h].x) + bf16_hi(qr[h].x)) + (bf16_lo(qr[h].y) + bf16_hi(qr[h].y))) +
            ((bf16_lo(qr[h].z) + bf16_hi(qr[h].z)) + (bf16_lo(qr[h].w) + bf16_hi(qr[h].w)));
}

template <int D, int G>
__device__ __forceinline__ void anchor_query_load(const FfdArgs& a, size_t hq0, int off,
                                                  u32x4 (&qr)[G]) {
  const uint16_t* qp = a.q + hq0 * D + off;
#pragma unroll
  for (int h = 0; h < G; ++h) qr[h] = ld16(qp + (size_t)h * D);
}

template <int D, int G>
__device__ __forceinline__ void anchor_query(const FfdArgs& a, size_t hq0, int off,
                                             u32x4 (&qr)[G], float (&ql)[G]) {
  anchor_query_load<D, G>(a, hq0, off, qr);
  query_sums<G>(qr, ql);
}

// Pseudo-maximum (FFD digest, section 4): for every query head of
// (sequence b, kv-head kvh), the largest refined score over the anchor
// positions -- the first n_sink and the last n_local positions -- and the
// lowest anchor position attaining it, in raw dot-product units.  Run by a
// whole workgroup, 16 lanes per anchor row; every thread receives the result.
// qr may still be in flight: its sums are formed after the anchor rows'
// loads are issued, so both share one memory latency.
template <int D, int G>
__device__ __forceinline__ void anchor_best(const FfdArgs& a, int b, int kvh,
                                            const u32x4 (&qr)[G],
                                            float (&s_best)[kWaves][G], int (&s_bidx)[kWaves][G],
                                            float (&out_best)[G], int (&out_pos)[G]) {
  using Gm = Geo<uint16_t, D>;
  constexpr int LPT = Gm::kLpt, TPL = Gm::kTpl;
  constexpr int NG = D / 32;
  constexpr int CW = D / 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
  const int grp = lane / LPT, col = lane % LPT;
  const int L = a.L;
  const size_t rbase = ((size_t)b * a.Hkv + kvh) * (size_t)L;
  const uint32_t* codes = a.codes;
  const uint16_t* zs = a.zs;
  const int8_t* res = a.res;
  const uint16_t* rsa = a.rs;
  const int n_sk = min(a.n_sink, L);
  const int loc0 = max(n_sk, L - a.n_local);
  const int na = n_sk + (L - loc0);
  float best[G];
  int bidx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { best[h] = kNegInf; bidx[h] = 0x7fffffff; }
  // All loads of up to NIT rounds (kWaves * TPL anchors each) are issued
  // before any arithmetic: one memory latency instead of one per round.
  // The first pass is peeled out of the loop (na >= 1 always) so that its
  // loads are issued before the query sums wait for qr.
  constexpr int NIT = 8;
  const int gi = col / 4;  // 8 dims per lane, 4 lanes per group
  auto pass = [&](int kb) {
    uint32_t w[NIT], zsb[NIT];
    u32x2 rr[NIT];
    uint32_t rsb[NIT];
    int pos[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int k = min(kb + (it * kWaves + wave) * TPL + grp, na - 1);
      pos[it] = k < n_sk ? k : loc0 + (k - n_sk);
      const size_t row = rbase + pos[it];
      w[it] = codes[row * CW + col / 2];
      zsb[it] = *reinterpret_cast<const uint32_t*>(zs + (row * NG + gi) * 2);
      rr[it] = *reinterpret_cast<const u32x2*>(res + row * D + col * 8);
      rsb[it] = rsa[row * NG + gi];
    }
    // keep the scheduler from pulling conversions of early loads in among
    // the later ones (each would wait for the loads issued before it)
    __builtin_amdgcn_sched_barrier(0);
    float ql[G];
    query_sums<G>(qr, ql);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const bool valid = kb + (it * kWaves + wave) * TPL + grp < na;
      const float z = half_to_float(zsb[it] & 0xFFFF), st = half_to_float(zsb[it] >> 16);
      float corr[G];
      residual_dot<G>(rr[it], half_to_float(rsb[it]), qr, ql, corr);
      const int p0 = 4 * (col & 1);
      const uint32_t k0p = code_pair(w[it], p0), k1p = code_pair(w[it], p0 + 1);
      const uint32_t k2p = code_pair(w[it], p0 + 2), k3p = code_pair(w[it], p0 + 3);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = dot2_bf16(qr[h].x, k0p, 0.f);
        float y = dot2_bf16(qr[h].y, k1p, 0.f);
        x = dot2_bf16(qr[h].z, k2p, x);
        y = dot2_bf16(qr[h].w, k3p, y);
        const float part = fmaf(fmaf(-4.f, st, z), ql[h], st * (x + y)) + corr[h];
        const float sc = group_sum<LPT>(part);
        if (valid && (sc > best[h] || (sc == best[h] && pos[it] < bidx[h]))) {
          best[h] = sc;
          bidx[h] = pos[it];
        }
      }
    }
  };
  pass(0);
  for (int kb = kWaves * TPL * NIT; kb < na; kb += kWaves * TPL * NIT) pass(kb);
  // (largest score, then lowest position) over the wave's lanes, by pair
  // exchanges; the order is total, so both lanes of a pair agree
  auto argmax_step = [&](auto off_tag) {
    constexpr int OFF = decltype(off_tag)::value;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float b0, b1, i0, i1;
      lane_pair<OFF>(best[h], b0, b1);
      lane_pair<OFF>(__int_as_float(bidx[h]), i0, i1);
      const int j0 = __float_as_int(i0), j1 = __float_as_int(i1);
      const bool second = b1 > b0 || (b1 == b0 && j1 < j0);
      best[h] = second ? b1 : b0;
      bidx[h] = second ? j1 : j0;
    }
  };
  if constexpr (LPT <= 4) argmax_step(std::integral_constant<int, 4>{});
  if constexpr (LPT <= 8) argmax_step(std::integral_constant<int, 8>{});
  if constexpr (LPT <= 16) argmax_step(std::integral_constant<int, 16>{});
  argmax_step(std::integral_constant<int, 32>{});
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { s_best[wave][h] = best[h]; s_bidx[wave][h] = bidx[h]; }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float bb = s_best[0][h];
    int bi = s_bidx[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const float ob = s_best[w][h];
      const int oi = s_bidx[w][h];
      if (ob > bb || (ob == bb && oi < bi)) { bb = ob; bi = oi; }
    }
    out_best[h] = bb;
    out_pos[h] = bi;
  }
}

// Pseudo-maximum kernel: one workgroup per (sequence, kv-head) runs
// anchor_best and leaves m^ (raw units) and j* per query head in the
// workspace for the FFD kernel (and m^ scaled in pseudo_max, if requested).
template <int D, int G>
__global__ __launch_bounds__(kThreads) void ffd_anchor_kernel(FfdArgs a) {
  using Gm = Geo<uint16_t, D>;
  constexpr int VEC = Gm::kVec, LPT = Gm::kLpt;
  __shared__ float s_best[kWaves][G];
  __shared__ int s_bidx[kWaves][G];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), col = lane % LPT;
  const int kvh = blockIdx.x % a.Hkv, b = blockIdx.x / a.Hkv;
  const size_t hq0 = (size_t)b * a.Hq + (size_t)kvh * G;
  u32x4 qr[G];
  anchor_query_load<D, G>(a, hq0, col * VEC, qr);
  float bb[G];
  int bi[G];
  anchor_best<D, G>(a, b, kvh, qr, s_best, s_bidx, bb, bi);
  if (tid == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      a.anchor_max[hq0 + h] = bb[h];
      a.anchor_pos[hq0 + h] = bi[h];
      if (a.pseudo_max != nullptr) a.pseudo_max[hq0 + h] = bb[h] * a.scale;
    }
  }
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

template <int D, int G>
__global__ __launch_bounds__(kThreads) void ffd_kernel(FfdArgs a) {
  using Gm = Geo<uint16_t, D>;
  constexpr int VEC = Gm::kVec, LPT = Gm::kLpt, TPL = Gm::kTpl;
  constexpr int kNb = kRefineRows;   // rows per slot per batch in the refine
  constexpr int NG = D / 32;         // quantisation groups per position
  constexpr int TPS = kWave / NG;    // positions per wave step in the scan
  constexpr int CW = D / 16;         // code words per position

  extern __shared__ __align__(16) unsigned char s_dyn[];
  float (*s_scan)[G] = reinterpret_cast<float (*)[G]>(s_dyn);
  uint8_t* s_mask = s_dyn + ffd_lds_mask_off<G>(a.chunk);
  uint16_t* s_list = reinterpret_cast<uint16_t*>(s_dyn + ffd_lds_list_off<G>(a.chunk));
  __shared__ int s_cnt[kWaves];
  __shared__ CombineLds<G, D> s_cmb;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
  const int grp = lane / LPT, col = lane % LPT;
  const int c = blockIdx.x % a.nc;
  const int bk = blockIdx.x / a.nc;
  const int kvh = bk % a.Hkv, b = bk / a.Hkv;
  const int L = a.L;
  const int c0 = c * a.chunk, c1 = min(c0 + a.chunk, L), n = c1 - c0;
  const size_t bkv = (size_t)b * a.Hkv + kvh;
  const size_t rbase = bkv * (size_t)L;  // row index of position 0
  const uint32_t* codes = a.codes;
  const uint16_t* zs = a.zs;
  const int8_t* res = a.res;
  const uint16_t* rsa = a.rs;
  const char* vb = reinterpret_cast<const char*>(a.v) + rbase * Gm::kRow;
  const size_t hq0 = (size_t)b * a.Hq + (size_t)kvh * G;

  // Query slices of the 16-lane (row) layout, and their partial sums.
  u32x4 qr[G];
  float ql[G];
  anchor_query<D, G>(a, hq0, col * VEC, qr, ql);

  // ---- 0. pseudo-maximum and its anchor ----
  float thr[G];
  int jst[G];
  // computed once per (sequence, kv-head) by ffd_anchor_kernel (scoring the
  // anchors in every chunk's workgroup instead measured 14-15 us slower)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    thr[h] = a.anchor_max[hq0 + h] - a.delta_raw;
    jst[h] = a.anchor_pos[hq0 + h];
  }

  // ---- 1. 2-bit scan of the chunk: scores and candidate masks into LDS ----
  if constexpr (D == 128 && (G == 4 || G == 8)) {
    // On the matrix cores.  For each 16-row tile of heads 4*tt .. 4*tt+3 the
    // four quantisation groups are stacked block-diagonally: row i = 4g + e
    // is (group g, head 4*tt + e), and k-step t of v_mfma_f32_16x16x32_bf16
    // gives lane quad g the 8 dims 32g + 8t .. +8 of group g.  A = query
    // (zero outside the row's own group), B = codes of 16 positions as exact
    // bf16 4 + c, so C[(g, h)][pos] = sum over group g of q_h,i (4 + c_i).
    // Lane (pos n16, quad g) loads that position's codes and (zero, step) of
    // group g and receives C for exactly that group: one fma per head gives
    // the group's part of the score, two shuffles sum the four groups.
    constexpr int NT = G / 4;
    constexpr int TB = kScanTiles;            // 16-position tiles per load round
    const int n16 = lane & 15, qg = lane >> 4;
    u32x4 qa[NT][4];
    float qsum[NT][4];
    stacked_query<G>(a.q + hq0 * D, lane, qa, qsum);
    for (int p0 = wave * 16 * TB; p0 < n; p0 += kWaves * 16 * TB) {
      u32x2 cw[TB];
      uint32_t zz[TB];
#pragma unroll
      for (int bt = 0; bt < TB; ++bt) {
        const int jr = min(p0 + 16 * bt + n16, n - 1);
        const size_t row = rbase + c0 + jr;
        cw[bt] = ffd_load(reinterpret_cast<const u32x2*>(codes + row * CW + 2 * qg));
        zz[bt] = ffd_load(reinterpret_cast<const uint32_t*>(zs + (row * NG + qg) * 2));
      }
#pragma unroll
      for (int bt = 0; bt < TB; ++bt) {
        const int jr = p0 + 16 * bt + n16;
        u32x4 bk[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t w = t < 2 ? cw[bt].x : cw[bt].y;
          const int pb = 4 * (t & 1);
          bk[t] = u32x4{code_pair(w, pb), code_pair(w, pb + 1), code_pair(w, pb + 2),
                        code_pair(w, pb + 3)};
        }
        const float z = half_to_float(zz[bt] & 0xFFFF), st = half_to_float(zz[bt] >> 16);
        const float zb = fmaf(-4.f, st, z);
        uint32_t bits = 0;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t)
            cc = mfma_16x16x32(qa[tt][t], bk[t], cc);
          float sc[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sc[e] = fmaf(zb, qsum[tt][e], st * cc[e]);
            sc[e] = pair_sum<32>(pair_sum<16>(sc[e]));
            const int h = 4 * tt + e;
            const bool cand = (sc[e] >= thr[h]) || (c0 + jr == jst[h]);
            bits |= cand ? (1u << h) : 0u;
          }
          if (qg == 0 && jr < n)
            *reinterpret_cast<f32x4*>(&s_scan[jr][4 * tt]) = f32x4{sc[0], sc[1], sc[2], sc[3]};
        }
        if (qg == 0 && jr < n) s_mask[jr] = (uint8_t)bits;
      }
    }
  } else {
    const int gi = lane % NG, tk = lane / NG;
    u32x4 qs[G][4];
    float qg[G];
    const uint16_t* qp = a.q + hq0 * D + gi * 32;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qg[h] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qs[h][j] = ld16(qp + (size_t)h * D + j * 8);
        qg[h] += (bf16_lo(qs[h][j].x) + bf16_hi(qs[h][j].x)) +
                 (bf16_lo(qs[h][j].y) + bf16_hi(qs[h][j].y)) +
                 (bf16_lo(qs[h][j].z) + bf16_hi(qs[h][j].z)) +
                 (bf16_lo(qs[h][j].w) + bf16_hi(qs[h][j].w));
      }
    }
    constexpr int kSteps = kScanSteps;
    for (int r0 = wave * TPS * kSteps; r0 < n; r0 += kWaves * TPS * kSteps) {
      u32x2 cw[kSteps];
      uint32_t zz[kSteps];
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const int jr = min(r0 + u * TPS + tk, n - 1);
        const size_t row = rbase + c0 + jr;
        cw[u] = ffd_load(reinterpret_cast<const u32x2*>(codes + row * CW + 2 * gi));
        zz[u] = ffd_load(reinterpret_cast<const uint32_t*>(zs + (row * NG + gi) * 2));
      }
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const int jr = r0 + u * TPS + tk;
        const float z = half_to_float(zz[u] & 0xFFFF), st = half_to_float(zz[u] >> 16);
        const float zb = fmaf(-4.f, st, z);
        uint32_t kp[16];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          kp[p] = code_pair(cw[u].x, p);
          kp[8 + p] = code_pair(cw[u].y, p);
        }
        uint32_t bits = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = 0.f, y = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x = dot2_bf16(qs[h][j].x, kp[4 * j + 0], x);
            y = dot2_bf16(qs[h][j].y, kp[4 * j + 1], y);
            x = dot2_bf16(qs[h][j].z, kp[4 * j + 2], x);
            y = dot2_bf16(qs[h][j].w, kp[4 * j + 3], y);
          }
          float sc = fmaf(zb, qg[h], st * (x + y));
          sc += dpp<kQuadXor1>(sc);
          if constexpr (NG == 4) sc += dpp<kQuadXor2>(sc);
          const bool cand = (sc >= thr[h]) || (c0 + jr == jst[h]);
          bits |= cand ? (1u << h) : 0u;
          if (jr < n && gi == (h % NG)) s_scan[jr][h] = sc;
        }
        if (jr < n && gi == 0) s_mask[jr] = (uint8_t)bits;
      }
    }
  }
  __syncthreads();

  // Candidate bitmask output (optional): word j/32, bit j%32, per head.
  if (a.cand_mask != nullptr) {
    const int nw = (n + 31) / 32;
    const size_t words = ((size_t)L + 31) / 32;
    for (int idx = tid; idx < G * nw; idx += kThreads) {
      const int h = idx / nw, wi = idx % nw;
      uint32_t word = 0;
      for (int k = 0; k < 32; ++k) {
        const int jr = wi * 32 + k;
        if (jr < n && ((s_mask[jr] >> h) & 1)) word |= 1u << k;
      }
      a.cand_mask[(hq0 + h) * words + (size_t)(c0 / 32) + wi] = word;
    }
  }

  // ---- 2. compaction of the group's candidate union ----
  int nu = 0;
  for (int r0 = 0; r0 < n; r0 += kThreads) {
    const int jr = r0 + tid;
    const bool u = jr < n && s_mask[jr] != 0;
    const unsigned long long bal = __ballot(u);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = nu, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      off += (w < wave) ? s_cnt[w] : 0;
      tot += s_cnt[w];
    }
    if (u) s_list[off + pre] = (uint16_t)jr;
    nu += tot;
    __syncthreads();
  }

  // ---- 3. refine + exact attention over the candidates ----
  if constexpr (D == 128 && (G == 4 || G == 8)) {
    // On the matrix cores, 16 candidates per tile (a wave takes tiles
    // wave, wave + 4, ...):
    //   residual: the same group-stacked tile as the scan, B = residual bytes
    //     as exact bf16 r + 128: C[(g, h)][cand] = sum_g q_h,i (r_i + 128),
    //     so the refinement is rs_g (C - 128 qsum_h,g), summed over g;
    //   softmax per head across the tile's 16 lanes (DPP), p in fp32;
    //   P V: p staged in LDS as [head][candidate] and read back as the A
    //     operand of v_mfma_f32_16x16x16_bf16 (rows = heads, split bf16
    //     hi + lo for fp32-level accuracy), V rows through an LDS tile read
    //     back transposed (ds_read_b64_tr_b16) as the B operand.
    constexpr int NT = G / 4;
    constexpr int VSTR = 2 * D + 8;   // LDS row stride of the V tile
    __shared__ __align__(16) unsigned char s_vt[kWaves][16 * VSTR];
    __shared__ __align__(16) float s_pb[kWaves][G][16];
    const int n16 = lane & 15, qg = lane >> 4;
    u32x4 qa[NT][4];
    float qsum[NT][4];
    stacked_query<G>(a.q + hq0 * D, lane, qa, qsum);
    unsigned char* lv = s_vt[wave];
    const int tr_off = (4 * qg + (n16 >> 2)) * VSTR + 8 * (n16 & 3);
    f32x4 o[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mh[G], lh[G];   // raw running maximum per head; this lane's part of l
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mh[h] = kNegInf;
      lh[h] = 0.f;
    }
    // Loads of a tile go through buffer descriptors of this chunk's residual,
    // step and V rows.  The next tile's residuals are requested as soon as
    // the current ones are unpacked and its V rows as soon as the current
    // ones are in LDS, so a tile's loads travel during the previous tile's
    // math without extra registers.  Slots past the candidate list (and the
    // whole tile after a wave's last) get an offset beyond the descriptor's
    // limit: the load is still issued, so every path has the same loads in
    // flight and the compiler's wait counts stay exact, but it reads zeros
    // without touching memory.
    const __amdgpu_buffer_rsrc_t rs_res = buffer_rsrc(res + (rbase + c0) * D, n * D);
    const __amdgpu_buffer_rsrc_t rs_rs = buffer_rsrc(rsa + (rbase + c0) * NG, n * NG * 2);
    const __amdgpu_buffer_rsrc_t rs_v = buffer_rsrc(vb + (size_t)c0 * Gm::kRow, n * Gm::kRow);
    auto res_issue = [&](int t0, u32x4& r0, u32x4& r1, uint32_t& rsh) {
      const int jn = t0 + n16;
      const int jr = s_list[min(jn, nu - 1)];
      const int off = jn < nu ? jr * D + 32 * qg : n * D;
      r0 = ld16_buf(rs_res, off);
      r1 = ld16_buf(rs_res, off + 16);
      rsh = __builtin_amdgcn_raw_buffer_load_b16(
          rs_rs, jn < nu ? (jr * NG + qg) * 2 : n * NG * 2, 0, kBufferNonTemporal);
    };
    auto v_issue = [&](int t0, u32x4 (&vr)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jj = t0 + 4 * i + qg;
        const int jv = s_list[min(jj, nu - 1)];
        vr[i] = ld16_buf(rs_v, jj < nu ? jv * Gm::kRow + 16 * n16 : n * Gm::kRow);
      }
    };
    u32x4 r0, r1;
    uint32_t rsh = 0;
    u32x4 vr[4];   // V rows of tile slots 4i + qg, 16 bytes at 16 * n16
    if (wave * 16 < nu) {
      res_issue(wave * 16, r0, r1, rsh);
      v_issue(wave * 16, vr);
    }
    for (int t0 = wave * 16; t0 < nu; t0 += kWaves * 16) {
      const int jn = t0 + n16;                      // this lane's candidate slot
      const int jr = s_list[min(jn, nu - 1)];
      const float rsf = half_to_float(rsh);
      const uint32_t mk = s_mask[jr];
      const bool valid = jn < nu;
      u32x4 bk[4];
      {
        const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x2 lo = residual_pairs(w[2 * t]), hi = residual_pairs(w[2 * t + 1]);
          bk[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
      }
      res_issue(t0 + kWaves * 16, r0, r1, rsh);
      float sh[G];   // refined raw scores of this lane's candidate
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) cc = mfma_16x16x32(qa[tt][t], bk[t], cc);
        const f32x4 sv = *reinterpret_cast<const f32x4*>(&s_scan[jr][4 * tt]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float corr = rsf * fmaf(-128.f, qsum[tt][e], cc[e]);
          corr = pair_sum<32>(pair_sum<16>(corr));
          const int h = 4 * tt + e;
          sh[h] = (valid && ((mk >> h) & 1u)) ? sv[e] + corr : kNegInf;
        }
      }
      // online softmax per head over the tile (all lanes of a 16-lane row
      // hold the same candidate set, every quad the same values)
      bool grow = false;
      float alpha[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(mh[h], group_max<16>(sh[h]));
        alpha[h] = (mn == mh[h]) ? 1.f : exp2_hw((mh[h] - mn) * a.c_log2);
        grow |= mn > mh[h];
        mh[h] = mn;
      }
      if (__any(grow)) {
#pragma unroll
        for (int h = 0; h < G; ++h) lh[h] *= alpha[h];
        // O row 4*qg + e is head 4*qg + e (rows >= G are padding)
        float ae[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ae[e] = 1.f;
#pragma unroll
          for (int h = e; h < G; h += 4) ae[e] = (h == 4 * qg + e) ? alpha[h] : ae[e];
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][e] *= ae[e];
      }
      float* pb = &s_pb[wave][0][0];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // exponent (s - m) c: exactly 0, p exactly 1, at the running maximum
        const float base = (mh[h] == kNegInf) ? 0.f : mh[h];
        const float p = exp2_hw((sh[h] - base) * a.c_log2);
        lh[h] += p;
        if ((h & 3) == qg) pb[h * 16 + n16] = p;
      }
      // A operand: lane (head row n16, quad q) takes p[n16][4q .. 4q+3]
      u32x2 ph = {0u, 0u}, pl = {0u, 0u};
      if (n16 < G) {
        const f32x4 pv = *reinterpret_cast<const f32x4*>(pb + n16 * 16 + 4 * qg);
        // hi = bf16(p), lo = bf16(p - hi), rounded to nearest even by the
        // hardware conversion (two values per instruction)
        uint32_t hb[2], lb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float x0 = pv[2 * j], x1 = pv[2 * j + 1];
          hb[j] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)x0, (__bf16)x1});
          lb[j] = __builtin_bit_cast(
              uint32_t, bf16x2_t{(__bf16)(x0 - __uint_as_float(hb[j] << 16)),
                                 (__bf16)(x1 - __uint_as_float(hb[j] & 0xFFFF0000u))});
        }
        ph = u32x2{hb[0], hb[1]};
        pl = u32x2{lb[0], lb[1]};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(lv + (4 * i + qg) * VSTR + 16 * n16) = vr[i];
      v_issue(t0 + kWaves * 16, vr);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const u32x2 vv = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                       (__attribute__((address_space(3))) s16x4_t*)(lv + tr_off + 32 * db)));
        o[db] = mfma_16x16x16(ph, vv, o[db]);
        o[db] = mfma_16x16x16(pl, vv, o[db]);
      }
    }
    // ---- 4. waves merge into one partial per query head ----
#pragma unroll
    for (int h = 0; h < G; ++h) lh[h] = group_sum<16>(lh[h]);
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * qg + e < G) s_cmb.acc[wave][4 * qg + e][16 * db + n16] = o[db][e];
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_cmb.ml[wave][h][0] = (mh[h] == kNegInf) ? kNegInf : mh[h] * a.c_log2;
        s_cmb.ml[wave][h][1] = lh[h];
      }
    }
    __syncthreads();
    const size_t prow0 = hq0 * a.nc + c;
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int h = idx / D, dd = idx % D;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_cmb.ml[w][h][0]);
      float ov = 0.f, ls = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = exp2_diff(s_cmb.ml[w][h][0], M);
        ov = fmaf(wt, s_cmb.acc[w][h][dd], ov);
        ls = fmaf(wt, s_cmb.ml[w][h][1], ls);
      }
      const size_t prow = prow0 + (size_t)h * a.nc;
      a.o_part[prow * D + dd] = ov;
      if (dd == 0) {
        a.ml_part[prow * 2] = M;
        a.ml_part[prow * 2 + 1] = ls;
      }
    }
    return;
  }
  float acc[G][VEC], m[G], l[G];
  state_reset<G, VEC>(acc, m, l);
  const int per = (((nu + kWaves - 1) / kWaves) + TPL - 1) / TPL * TPL;
  const int t_beg = wave * per, t_end = min(t_beg + per, nu);
  for (int t0 = t_beg; t0 < t_end; t0 += kNb * TPL) {
    int jr[kNb];
    u32x2 rr[kNb];
    uint32_t rsb[kNb];
    u32x4 vr[kNb];
#pragma unroll
    for (int i = 0; i < kNb; ++i) {
      jr[i] = s_list[min(t0 + i * TPL + grp, t_end - 1)];
      const size_t row = rbase + c0 + jr[i];
      rr[i] = ffd_load(reinterpret_cast<const u32x2*>(res + row * D + col * 8));
      rsb[i] = rsa[row * NG + col / 4];
    }
#pragma unroll
    for (int i = 0; i < kNb; ++i)
      vr[i] = ffd_load(reinterpret_cast<const u32x4*>(vb + (size_t)(c0 + jr[i]) * Gm::kRow +
                                                      (size_t)col * 16));
    float s[kNb][G];
#pragma unroll
    for (int i = 0; i < kNb; ++i) {
      float corr[G];
      residual_dot<G>(rr[i], half_to_float(rsb[i]), qr, ql, corr);
      const uint32_t mk = s_mask[jr[i]];
      const bool valid = t0 + i * TPL + grp < t_end;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sc = s_scan[jr[i]][h] + group_sum<LPT>(corr[h]);
        s[i][h] = (valid && ((mk >> h) & 1)) ? sc : kNegInf;
      }
    }
    online_update<uint16_t, G, VEC, kNb>(s, vr, a.c_log2, acc, m, l);
  }
  state_to_log2<G>(m, a.c_log2);

  // ---- 4. one partial per query head ----
  combine_store<G, D, VEC, LPT>(s_cmb, acc, m, l, a.o_part, a.ml_part,
                                hq0 * a.nc + c, (size_t)a.nc);
}

// Packer: one thread per (position, 32-dim group).  Every step in fp32 with
// round-to-nearest-even, in the order the format defines (see fd.h).
template <int D>
__global__ __launch_bounds__(kThreads) void ffd_pack_kernel(FfdPackArgs a) {
  constexpr int NG = D / 32;
  const int span = a.t_end - a.t_begin;
  const size_t total = (size_t)a.B * a.Hkv * span * NG;
  const size_t gid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= total) return;
  const int gi = (int)(gid % NG);
  const size_t pt = gid / NG;
  const int t = a.t_begin + (int)(pt % span);
  const size_t bkv = pt / span;
  const size_t row = bkv * (size_t)a.Lcap + t;

  float x[32];
  const u32x4* src = reinterpret_cast<const u32x4*>(a.k + row * D + gi * 32);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 w = src[j];
    x[8 * j + 0] = bf16_lo(w.x); x[8 * j + 1] = bf16_hi(w.x);
    x[8 * j + 2] = bf16_lo(w.y); x[8 * j + 3] = bf16_hi(w.y);
    x[8 * j + 4] = bf16_lo(w.z); x[8 * j + 5] = bf16_hi(w.z);
    x[8 * j + 6] = bf16_lo(w.w); x[8 * j + 7] = bf16_hi(w.w);
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
  const _Float16 z16 = (_Float16)mn;
  const _Float16 s16 = (_Float16)((mx - mn) / 3.0f);
  const float z = (float)z16, st = (float)s16;
  uint32_t code[32];
  float r[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float cf = 0.f;
    if (st != 0.f) cf = fminf(fmaxf(__builtin_rintf((x[i] - z) / st), 0.f), 3.f);
    code[i] = (uint32_t)cf;
    r[i] = x[i] - fmaf(st, cf, z);
    amax = fmaxf(amax, fabsf(r[i]));
  }
  const _Float16 rs16 = (_Float16)(amax / 127.0f);
  const float rsf = (float)rs16;
  uint32_t rb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rb[j] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float q = 0.f;
    if (rsf != 0.f) q = fminf(fmaxf(__builtin_rintf(r[i] / rsf), -127.f), 127.f);
    rb[i / 4] |= ((uint32_t)(int)q & 0xFFu) << (8 * (i % 4));
  }
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    w0 |= (code[2 * p] << (2 * p)) | (code[2 * p + 1] << (16 + 2 * p));
    w1 |= (code[16 + 2 * p] << (2 * p)) | (code[17 + 2 * p] << (16 + 2 * p));
  }
  *reinterpret_cast<u32x2*>(a.codes + row * (D / 16) + 2 * gi) = u32x2{w0, w1};
  *reinterpret_cast<uint32_t*>(a.zs + (row * NG + gi) * 2) =
      (uint32_t)__builtin_bit_cast(uint16_t, z16) |
      ((uint32_t)__builtin_bit_cast(uint16_t, s16) << 16);
  u32x4* dst = reinterpret_cast<u32x4*>(a.res + row * D + gi * 32);
  dst[0] = u32x4{rb[0], rb[1], rb[2], rb[3]};
  dst[1] = u32x4{rb[4], rb[5], rb[6], rb[7]};
  a.rs[row * NG + gi] = __builtin_bit_cast(uint16_t, rs16);
}

hipError_t launch_ffd(int D, int G, const FfdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)a.B * a.Hkv * a.nc)), block(kThreads);
#define FD_FFD_CASE(DD, GG)                                                          \
  if (D == DD && G == GG) {                                                          \
    hipLaunchKernelGGL((ffd_anchor_kernel<DD, GG>), dim3((unsigned)(a.B * a.Hkv)), block, 0, \
                       s, a);                                                        \
    hipError_t e = hipGetLastError();                                                \
    if (e != hipSuccess) return e;                                                   \
    hipLaunchKernelGGL((ffd_kernel<DD, GG>), grid, block, ffd_lds_bytes<GG>(a.chunk), s, a); \
    return hipGetLastError();                                                        \
  }
  FD_FFD_CASE(64, 1) FD_FFD_CASE(64, 2) FD_FFD_CASE(64, 4) FD_FFD_CASE(64, 8)
  FD_FFD_CASE(128, 1) FD_FFD_CASE(128, 2) FD_FFD_CASE(128, 4) FD_FFD_CASE(128, 8)
#undef FD_FFD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_ffd_pack(int D, const FfdPackArgs& a, hipStream_t s) {
  const size_t total = (size_t)a.B * a.Hkv * (a.t_end - a.t_begin) * (D / 32);
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads)), block(kThreads);
  if (D == 64) hipLaunchKernelGGL((ffd_pack_kernel<64>), grid, block, 0, s, a);
  else if (D == 128) hipLaunchKernelGGL((ffd_pack_kernel<128>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fdk
