// FFD sparse decode, streamed by single wavefronts (d = 128, G = 4 or 8):
// the 2-bit scan, top-delta selection, 8-bit refine and exact attention of
// the "Faster Than Flash" digest (longzhangge.com, sections 3, 5 and 6,
// Fig. 2) for one chunk per wavefront, fused, with no intermediate written
// to memory, the pseudo-maximum m^ and its anchor j* (section 4) included.
//
// A wavefront owns one unit = (sequence, kv-head, chunk).  It first scores
// the anchor positions (the first n_sink and the last n_local positions of
// its sequence) with the refined keys, as below, for m^ and j* -- split
// over the four waves of the workgroup when they share a (sequence,
// kv-head), the kernel's one barrier -- then walks its chunk in steps of
// kStep positions:
//   * Scan.  Codes and (zero, step) of a step's 8 tiles of 16 positions come
//     through buffer loads (one lane offset plus an immediate per tile).
//     Codes become exact fp16 subnormals c 2^(2i-24) with one mask per pair
//     of dims (i = the pair's place in its 32-bit word) and the query fp16
//     after exact power-of-two scalings; v_mfma_f32_16x16x32_f16 with the
//     query groups stacked block-diagonally gives each lane (position n,
//     quad g) the group-g dot products of heads 4tt .. 4tt+3, and a
//     transposed reduction over the four quads (two v_permlane32_swap, one
//     v_permlane16_swap, each adding) leaves lane (n, g) the full scan score
//     of head 4tt + g: three exchanges instead of the eight a full
//     reduction per head needs.
//   * Selection.  s~ >= m^ - delta (or the position is j*) per lane; one
//     ballot per head tile gives every head's 16 bits, and their union (in
//     scalar registers) the positions that need a refine.  Those positions
//     and their per-head scan scores (-inf where a head did not select the
//     position) are appended to a ring in this wave's LDS.
//   * Refine + attend, pairs of up to 32 ring entries (two tiles of 16),
//     while the next steps' scan loads are in flight: residual bytes as
//     exact fp16 subnormals (r + 128) 2^-24 (one byte permute per pair of
//     dims) in the same group-stacked tile (refinement = rs_g 2^24
//     (C - 2^-17 qsum), reduced the same transposed way), online softmax
//     per head over the pair, P V on
//     v_mfma_f32_16x16x32_bf16 over both tiles with p split bf16 hi + lo and
//     the candidates' V rows read back transposed from LDS.  The next
//     pair's loads are issued as soon as the current pair's registers are
//     free.  After each half-step the entries appended before it are
//     refined; the last entries after the walk.
//   * One partial (O, m, l) per query head at the end; the chunks merge in
//     the common log-sum-exp kernel.
#include "ffd_common.hpp"

namespace fdk {

namespace {
// 16-position scan tiles per step (two steps of scan loads are in flight:
// fewer for G = 8, whose query operands take twice the registers)
template <int G>
constexpr int scan_tiles() { return G == 4 ? 8 : 4; }
// ring entries per wave: at most two steps of entries wait for a refine
constexpr int kRing = 256;
// LDS row stride of a V tile (bytes): row r starts 8 r banks on, so the
// transposing 8-byte reads never share a bank (an 8-byte padding had 4x
// conflicts)
constexpr int kVStr = 2 * 128 + 32;
}  // namespace

// out = lanes' sum of x over the quad pair {g, g ^ 2} for lanes of quads 0
// and 1 (x) or 2 and 3 (y): v_permlane32_swap hands each lane both values.
__device__ __forceinline__ float swap_add32_pair(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_add16_pair(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane (n, g) holds t[e] = group g's part for head e of a 4-head tile at
// column n; returns the sum over the four groups for head g:
// (t(g) + t(g ^ 2)) + (t(g ^ 1) + t(g ^ 3)), the same order in every lane.
__device__ __forceinline__ float quad_transpose_sum(const float (&t)[4]) {
  const float y0 = swap_add32_pair(t[0], t[2]);   // quads 0, 1: head 0; quads 2, 3: head 2
  const float y1 = swap_add32_pair(t[1], t[3]);   // quads 0, 1: head 1; quads 2, 3: head 3
  return swap_add16_pair(y0, y1);                 // quad g: head g
}

__device__ __forceinline__ float lane_value(float x, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}

// Two waves share each SIMD (two workgroups per compute unit), and the
// hardware issues for the older one first: with equal work the younger
// workgroup finished 8 us (peaked scores) to 28 us (iid) after the older on
// every compute unit, then ran alone at one wave per SIMD.  Each wave
// therefore raises its issue priority (s_setprio) in alternate 5.12 us
// slices of the 100 MHz clock, the two waves of a SIMD (hardware wave slots
// 0 and 1) in opposite slices: the end gap fell to 3 us (peaked) and 12 us
// (iid); iid 150.8 -> 148.9 us per call, peaked unchanged (same process,
// interleaved).
__device__ __forceinline__ void fair_share_priority(uint32_t slot) {
  const uint64_t t = __builtin_amdgcn_s_memrealtime();
  if ((((uint32_t)(t >> 9)) ^ slot) & 1u)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Registers of one scan step: tile t's codes and (zero, step) of position
// 16 t + n16, quantisation group qg.
template <int T>
struct ScanRegs {
  u32x2 cw[T];
  uint32_t zz[T];
};

// Registers of one refine pair (ring entries t0 .. t0 + 31, two tiles of 16):
// residual bytes and scale of entry t0 + 16 k + n16, group qg, and 16 bytes
// (at 16 n16) of the V rows of entries t0 + 16 k + 4 i + qg.
struct PairRegs {
  u32x4 r0[2], r1[2];
  uint32_t rs[2];
  u32x4 v[2][4];
};

// MASK: the candidate bitmask output is requested (a separate instantiation,
// so that the hot loop carries no mask code otherwise).
template <int G, bool MASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void ffd_wave_kernel(FfdArgs a) {
  constexpr int D = 128, NG = D / 32, CW = D / 16, NT = G / 4;
  constexpr int kTiles = scan_tiles<G>(), kStep = 16 * kTiles;
  static_assert(G == 4 || G == 8, "group-stacked tiles");
  static_assert(2 * kStep <= kRing, "two steps of entries fit in the ring");
  // ring entries, then discard slots for the lanes of a tile that append
  // nothing (16 score rows, 64 positions), so that the appends are stores
  // on every lane and a scan step needs no branch
  __shared__ __align__(16) float s_sc[kWaves][kRing + 16][G];   // scan score per head (-inf: not selected)
  __shared__ int s_pos[kWaves][kRing + kWave];                   // position within the chunk
  __shared__ __align__(16) unsigned char s_vt[kWaves][2][16 * kVStr];
  __shared__ __align__(16) float s_pb[kWaves][G][32];
  __shared__ float s_am[kWaves][G];   // anchors: each wave's best score per head
  __shared__ int s_aj[kWaves][G];     // and its lowest position

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int n16 = lane & 15, qg = lane >> 4;
  const int unit = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kWaves + wave);
  if (unit >= a.B * a.Hkv * a.nc) return;
  const int c = unit % a.nc, bk = unit / a.nc;
  const int kvh = bk % a.Hkv, b = bk / a.Hkv;
  const int c0 = c * a.chunk, n = min(c0 + a.chunk, a.L) - c0;
  const size_t rbase = ((size_t)b * a.Hkv + kvh) * (size_t)a.L + c0;   // row of position c0
  const size_t hq0 = (size_t)b * a.Hq + (size_t)kvh * G;

  // The query as fp16, scaled by pw = 2^k (exact; see stacked_query_f16):
  // every score below is pw times the unscaled one, bit for bit, so
  // thresholds and maxima live in the scaled units and the softmax exponent
  // takes c log2 e / pw.  Set up after the first anchor and scan loads are
  // issued (below).
  float pw = 1.f, ipw = 1.f, cl2 = a.c_log2;
  u32x4 qa[NT][4], qs[NT][4];
  float qsum[NT][4];
  // this lane's heads 4 tt + qg: threshold m^ - delta and j* (within the
  // chunk), set from the anchors below
  float thr[NT];
  int jst[NT];
  // ---- operands and dot products shared by the anchors, the scan and the
  // refine.  Codes of a (position, group): k-step k takes pairs 4 (k % 2)
  // .. +3 of word k / 2, each half c 2^(2i-24); the products with qs sum to
  // 2^-24 pw sum q c, so the group's part of the 2-bit score of head
  // 4 tt + qg is z qsum + 2^24 st C, summed over the groups by the
  // transposed reduction ----
  auto code_operands = [&](const u32x2& cwv, u32x4 (&bq)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) bq[k] = code_operand_f16(k < 2 ? cwv.x : cwv.y, k & 1);
  };
  auto scan_scores = [&](const u32x4 (&bq)[4], uint32_t zzv, float (&sc)[NT]) {
    const float z = half_to_float(zzv & 0xFFFF), st = half_to_float(zzv >> 16) * 0x1p24f;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k) cc = mfma_16x16x32_f16(qs[tt][k], bq[k], cc);
      float part[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) part[e] = fmaf(z, qsum[tt][e], st * cc[e]);
      sc[tt] = quad_transpose_sum(part);
    }
  };
  // residual bytes of a (position, group) as exact fp16 (r + 128) 2^-24,
  // and the refinement rs_g sum q r = rs_g 2^24 (C - 2^-17 qsum) summed over
  // the groups (C = 2^-24 sum pw q (r + 128))
  auto residual_operands = [&](const u32x4& ra, const u32x4& rb, u32x4 (&bq)[4]) {
    const uint32_t w[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x2 lo = residual_pairs_f16(w[2 * t]), hi = residual_pairs_f16(w[2 * t + 1]);
      bq[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  };
  auto refinement = [&](const u32x4 (&bq)[4], float rsf, float (&corr)[NT]) {
    const float rs24 = rsf * 0x1p24f;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) cc = mfma_16x16x32_f16(qa[tt][t], bq[t], cc);
      float part[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) part[e] = rs24 * fmaf(-0x1p-17f, qsum[tt][e], cc[e]);
      corr[tt] = quad_transpose_sum(part);
    }
  };

  // ---- buffer descriptors of the chunk ----
  const char* codes_c = reinterpret_cast<const char*>(a.codes + rbase * CW);
  const char* zs_c = reinterpret_cast<const char*>(a.zs + rbase * NG * 2);
  const __amdgpu_buffer_rsrc_t rs_res = buffer_rsrc(a.res + rbase * D, n * D);
  const __amdgpu_buffer_rsrc_t rs_rs = buffer_rsrc(a.rs + rbase * NG, n * NG * 2);
  const __amdgpu_buffer_rsrc_t rs_v = buffer_rsrc(a.v + rbase * D, n * D * 2);

  // ---- scan loads of step s (positions s kStep ..), no memory access for
  // positions at or past n ----
  const int lane_c = n16 * (CW * 4) + 8 * qg, lane_z = n16 * (NG * 4) + 4 * qg;
  auto scan_issue = [&](ScanRegs<kTiles>& R, int s) __attribute__((always_inline)) {
    const int p0 = s * kStep, cnt = max(0, min(n - p0, kStep));
    const __amdgpu_buffer_rsrc_t rc =
        buffer_rsrc(codes_c + (size_t)min(p0, n) * (CW * 4), cnt * CW * 4);
    const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(zs_c + (size_t)min(p0, n) * (NG * 4), cnt * NG * 4);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      R.cw[t] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, lane_c + t * 16 * CW * 4, 0,
                                                      kBufferNonTemporal));
      R.zz[t] = __builtin_amdgcn_raw_buffer_load_b32(rz, lane_z + t * 16 * NG * 4, 0,
                                                     kBufferNonTemporal);
    }
  };

  // ---- refine loads of the pair at ring position t0.  An entry at or
  // past lim gets bit 30 in its offset, beyond every descriptor's limit:
  // the load is issued on every path (so the compiler's wait counts stay
  // exact) but reads zeros without touching memory.  The flag is or-ed into
  // the offset, not selected, so that the ring reads are unconditional (a
  // select lets the compiler branch around each read, serialising them).
  // Residuals first: they are needed first ----
  constexpr int kOob = 1 << 30;
  float* const sc_w = &s_sc[wave][0][0];
  int* const pos_w = s_pos[wave];
  auto res_issue = [&](PairRegs& P, int t0, int lim) __attribute__((always_inline)) {
    int jr[2], oob[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int jn = t0 + 16 * k + n16;
      jr[k] = pos_w[jn & (kRing - 1)];
      oob[k] = jn < lim ? 0 : kOob;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int off = (jr[k] * D + 32 * qg) | oob[k];
      P.r0[k] = ld16_buf(rs_res, off);
      P.r1[k] = ld16_buf(rs_res, off + 16);
      P.rs[k] = __builtin_amdgcn_raw_buffer_load_b16(rs_rs, ((jr[k] * NG + qg) * 2) | oob[k], 0,
                                                     kBufferNonTemporal);
    }
  };
  auto v_issue = [&](PairRegs& P, int t0, int lim) __attribute__((always_inline)) {
    int off[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jj = t0 + 16 * k + 4 * i + qg;
        off[k][i] = (pos_w[jj & (kRing - 1)] * (D * 2) + 16 * n16) | (jj < lim ? 0 : kOob);
      }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) P.v[k][i] = ld16_buf(rs_v, off[k][i]);
  };

  // ---- attention state: O rows 4 qg + e (= heads; rows >= G are padding),
  // dims 16 db + n16; this lane's heads 4 tt + qg: running maximum (raw
  // dot units) and its part of l ----
  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mh[NT], lh[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    mh[tt] = kNegInf;
    lh[tt] = 0.f;
  }
  unsigned char* lv0 = s_vt[wave][0];
  unsigned char* lv1 = s_vt[wave][1];
  const int tr_off = (4 * qg + (n16 >> 2)) * kVStr + 8 * (n16 & 3);
  float* pb = &s_pb[wave][0][0];

  // One refine pair: entries t0 .. t0 + 31 valid below lim, loads in P.
  // Issues the loads of the next pair (at nx, valid below nlim) into P as
  // soon as each part of P is consumed.
  auto refine_pair = [&](PairRegs& P, int t0, int lim, int nx, int nlim) __attribute__((always_inline)) {
    float sh[2][NT];   // refined raw score of this lane's entries for head 4 tt + qg
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x4 bq[4];
      residual_operands(P.r0[k], P.r1[k], bq);
      float corr[NT];
      refinement(bq, half_to_float(P.rs[k]), corr);
      const int jn = t0 + 16 * k + n16;
      const int idx = jn & (kRing - 1);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const float sv = sc_w[idx * G + 4 * tt + qg];
        sh[k][tt] = jn < lim ? sv + corr[tt] : kNegInf;
      }
    }
    res_issue(P, nx, nlim);
    // online softmax per head over the pair (the 16 lanes of a quad hold one
    // head's entries, two per lane)
    bool grow = false;
    float alpha[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const float mn = fmaxf(mh[tt], group_max<16>(fmaxf(sh[0][tt], sh[1][tt])));
      alpha[tt] = (mn == mh[tt]) ? 1.f : exp2_hw((mh[tt] - mn) * cl2);
      grow |= mn > mh[tt];
      mh[tt] = mn;
    }
    if (__any(grow)) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) lh[tt] *= alpha[tt];
      // O row 4 qg + e is head h = 4 qg + e, whose factor sits in quad e of
      // head tile qg
      float ae[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ae[e] = lane_value(alpha[0], 16 * e);
        if constexpr (NT == 2) ae[e] = qg == 1 ? lane_value(alpha[1], 16 * e) : ae[e];
      }
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[db][e] *= ae[e];
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      // exponent (s - m) c: exactly 0, p exactly 1, at the running maximum
      const float base = (mh[tt] == kNegInf) ? 0.f : mh[tt];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float p = exp2_hw((sh[k][tt] - base) * cl2);
        lh[tt] += p;
        pb[(4 * tt + qg) * 32 + 16 * k + n16] = p;
      }
    }
    // A operand of the 16x16x32 P V over the pair: lane (head row n16, quad
    // q) takes p at positions 4q .. 4q+3 of both tiles (k = 8q + j stands
    // for position 4q + j % 4 of tile j / 4), split hi = bf16(p),
    // lo = bf16(p - hi)
    u32x4 ph = {0u, 0u, 0u, 0u}, pl = {0u, 0u, 0u, 0u};
    if (n16 < G) {
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const f32x4 pv = *reinterpret_cast<const f32x4*>(pb + n16 * 32 + 16 * k + 4 * qg);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float x0 = pv[2 * j], x1 = pv[2 * j + 1];
          const uint32_t h = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)x0, (__bf16)x1});
          hb[2 * k + j] = h;
          lb[2 * k + j] = __builtin_bit_cast(
              uint32_t, bf16x2_t{(__bf16)(x0 - __uint_as_float(h << 16)),
                                 (__bf16)(x1 - __uint_as_float(h & 0xFFFF0000u))});
        }
      }
      ph = u32x4{hb[0], hb[1], hb[2], hb[3]};
      pl = u32x4{lb[0], lb[1], lb[2], lb[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(lv0 + (4 * i + qg) * kVStr + 16 * n16) = P.v[0][i];
      *reinterpret_cast<u32x4*>(lv1 + (4 * i + qg) * kVStr + 16 * n16) = P.v[1][i];
    }
    v_issue(P, nx, nlim);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const u32x2 v0 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (__attribute__((address_space(3))) s16x4_t*)(lv0 + tr_off + 32 * db)));
      const u32x2 v1 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (__attribute__((address_space(3))) s16x4_t*)(lv1 + tr_off + 32 * db)));
      const u32x4 vb = {v0.x, v0.y, v1.x, v1.y};
      o[db] = mfma_16x16x32(ph, vb, o[db]);
      o[db] = mfma_16x16x32(pl, vb, o[db]);
    }
  };

  // ---- scan of one step: scores, selection, ring append ----
  const size_t mask_words = ((size_t)a.L + 31) / 32;
  const uint32_t below = (1u << n16) - 1u;   // positions of the tile before this lane's
  int tail = 0;                              // ring entries written so far (wave-uniform)
  auto scan_step = [&](const ScanRegs<kTiles>& R, int s) __attribute__((always_inline)) {
    // every tile's scores first: no branch between the tiles, so the
    // compiler interleaves one tile's matrix products with another's vector
    // work (positions at or past n read zeros and are masked below)
    float sc[kTiles][NT];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      u32x4 bq[4];
      code_operands(R.cw[t], bq);
      scan_scores(bq, R.zz[t], sc[t]);
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int p0 = s * kStep + 16 * t;   // wave-uniform
      const int jr = p0 + n16;
      const uint64_t b_in = __builtin_amdgcn_ballot_w64(jr < n);
      bool sel[NT];
      uint64_t bal[NT];
      uint32_t uni = 0;   // positions of the tile selected by any head (wave-uniform)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const bool hit = sc[t][tt] >= thr[tt], js = jr == jst[tt];
        sel[tt] = (jr < n) & (hit | js);
        bal[tt] = (__builtin_amdgcn_ballot_w64(hit) | __builtin_amdgcn_ballot_w64(js)) & b_in;
        const uint64_t f = bal[tt] | (bal[tt] >> 32);
        uni |= (uint32_t)(f | (f >> 16)) & 0xFFFFu;
      }
      // lanes of appended positions write ring entry tail + (their rank in
      // the union); the others their discard slots
      const bool mine = (uni >> n16) & 1u;
      const int idx = mine ? (tail + __builtin_popcount(uni & below)) & (kRing - 1) : kRing + n16;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) sc_w[idx * G + 4 * tt + qg] = sel[tt] ? sc[t][tt] : kNegInf;
      pos_w[(mine && qg == 0) ? idx : kRing + lane] = jr;
      tail += __builtin_popcount(uni);
      if (MASK && lane < G && p0 < n) {
        // 16 bits per head and tile; chunks start at multiples of 32, so
        // tile t of the chunk is half-word c0 / 16 + s * kTiles + t of the row
        const uint64_t bb = (NT == 2 && lane >= 4) ? bal[NT - 1] : bal[0];
        uint16_t* mrow = reinterpret_cast<uint16_t*>(a.cand_mask + (hq0 + lane) * mask_words);
        mrow[(c0 >> 4) + s * kTiles + t] = (uint16_t)(bb >> (16 * (lane & 3)));
        // an odd tile count leaves the upper half of the last word: zero it
        if (p0 + 16 >= n && ((p0 >> 4) & 1) == 0) mrow[(c0 >> 4) + s * kTiles + t + 1] = 0;
      }
    }
  };

  // ---- the walk: step s scans with loads issued two steps earlier, then
  // refines the entries known before it (the first pair's loads were issued
  // at the end of step s - 1, so they travelled during this scan); one pair
  // is always in flight, at ring position `head` with limit `plim` ----
  const int nsteps = (n + kStep - 1) / kStep;
  ScanRegs<kTiles> sA, sB;
  PairRegs P;
  int head = 0, plim = 0;

  // ---- pseudo-maximum (FFD digest, section 4), while the first two scan
  // steps' loads travel: the refined scores of the anchor positions -- the
  // first n_sink and the last n_local positions, a set -- for this lane's
  // heads, computed as in the scan and the refine; m^ = their maximum and
  // j* the lowest position attaining it.  Every workgroup of a (sequence,
  // kv-head) reads the same anchor rows (cache-resident after the first)
  // and computes the same values.  A workgroup's units are consecutive
  // chunks: when its four waves share one (sequence, kv-head), wave w
  // scores the anchor tiles w, w + 4, ... and the four results meet in LDS
  // (the maximum with the lowest position is a total order, so the result
  // does not depend on the split); otherwise each wave scores all of them.
  // Anchor rows are loaded one tile ahead of the products ----
  {
    const int u_first = (int)blockIdx.x * kWaves;
    const bool share = u_first + kWaves <= a.B * a.Hkv * a.nc &&
                       u_first / a.nc == (u_first + kWaves - 1) / a.nc;   // workgroup-uniform
    const int t_step = share ? kWaves : 1;
    const int n_sk = min(a.n_sink, a.L), loc0 = max(n_sk, a.L - a.n_local);
    const int na = n_sk + (a.L - loc0);
    const size_t row0 = rbase - c0;   // row of position 0
    float mbest[NT];
    int jbest[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      mbest[tt] = kNegInf;
      jbest[tt] = 0x7fffffff;
    }
    struct AnchorRows {
      u32x2 cw;
      uint32_t zz;
      u32x4 ra, rb;
      uint32_t rs;
      int pos;
    };
    auto anchor_load = [&](int k0, AnchorRows& A) __attribute__((always_inline)) {
      const int k = min(k0 + n16, na - 1);
      A.pos = k < n_sk ? k : loc0 + (k - n_sk);
      const size_t row = row0 + A.pos;
      A.cw = *reinterpret_cast<const u32x2*>(a.codes + row * CW + 2 * qg);
      A.zz = *reinterpret_cast<const uint32_t*>(a.zs + (row * NG + qg) * 2);
      A.ra = ld16(a.res + row * D + 32 * qg);
      A.rb = ld16(a.res + row * D + 32 * qg + 16);
      A.rs = a.rs[row * NG + qg];
    };
    AnchorRows cur, nxt;
    const int k_first = share ? 16 * wave : 0;
    // the query, the first two anchor tiles and the first two scan steps,
    // requested in the order they are needed: the vector-memory counter
    // completes in issue order, so each wait covers only what came before
    // (the scan loads after the query's: at kernel start every wave
    // requests at once, and the query came back 1.5 us sooner so)
    u32x4 qraw[NT][4];
    query_load<G>(a.q + hq0 * D, lane, qraw);
    const int kst = 16 * t_step;   // anchor tiles k_first, k_first + kst, ...
    anchor_load(min(k_first, na - 1), cur);
    anchor_load(min(k_first + kst, na - 1), nxt);
    pw = stacked_query_f16<G>(qraw, lane, qa, qs, qsum);
    ipw = 1.f / pw;   // a power of two: exact
    cl2 = a.c_log2 * ipw;
    scan_issue(sA, 0);
    scan_issue(sB, 1);
    for (int k0 = k_first; k0 < na; k0 += kst) {   // wave-uniform
      u32x4 bq[4];
      code_operands(cur.cw, bq);
      float sc[NT], corr[NT];
      scan_scores(bq, cur.zz, sc);
      residual_operands(cur.ra, cur.rb, bq);
      refinement(bq, half_to_float(cur.rs), corr);
      const bool valid = k0 + n16 < na;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const float sh = sc[tt] + corr[tt];
        if (valid && (sh > mbest[tt] || (sh == mbest[tt] && cur.pos < jbest[tt]))) {
          mbest[tt] = sh;
          jbest[tt] = cur.pos;
        }
      }
      cur = nxt;
      if (k0 + 2 * kst < na) anchor_load(k0 + 2 * kst, nxt);   // wave-uniform
    }
    // (largest score, then lowest position) over the 16 lanes of a quad;
    // the order is total, so every lane ends with the same pair
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const float ob = __shfl_xor(mbest[tt], off);
        const int oj = __shfl_xor(jbest[tt], off);
        if (ob > mbest[tt] || (ob == mbest[tt] && oj < jbest[tt])) {
          mbest[tt] = ob;
          jbest[tt] = oj;
        }
      }
    }
    if (share) {
      if (n16 == 0) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          s_am[wave][4 * tt + qg] = mbest[tt];
          s_aj[wave][4 * tt + qg] = jbest[tt];
        }
      }
      __syncthreads();
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        mbest[tt] = s_am[0][4 * tt + qg];
        jbest[tt] = s_aj[0][4 * tt + qg];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
          const float ob = s_am[w][4 * tt + qg];
          const int oj = s_aj[w][4 * tt + qg];
          if (ob > mbest[tt] || (ob == mbest[tt] && oj < jbest[tt])) {
            mbest[tt] = ob;
            jbest[tt] = oj;
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      thr[tt] = mbest[tt] - a.delta_raw * pw;
      jst[tt] = jbest[tt] - c0;
      if (a.pseudo_max != nullptr && c == 0 && n16 == 0)
        a.pseudo_max[hq0 + 4 * tt + qg] = (mbest[tt] * ipw) * a.scale;
    }
  }

  res_issue(P, 0, 0);   // an empty pair: its loads read nothing
  v_issue(P, 0, 0);

  // hardware wave slot within the SIMD (HW_ID bits 3:0)
  const uint32_t wslot = __builtin_amdgcn_s_getreg((3 << 11) | 4) & 1u;
  auto refine_until = [&](int mark) __attribute__((always_inline)) {
    while (head < mark) {   // wave-uniform
      fair_share_priority(wslot);
      const int nx = min(head + 32, plim);
      refine_pair(P, head, plim, nx, tail);
      head = nx;
      plim = tail;
    }
    if (plim == head && tail > head) {
      // the pair in flight is empty but entries wait: reissue it
      res_issue(P, head, tail);
      v_issue(P, head, tail);
      plim = tail;
    }
  };
  // Both halves run on every trip (a step at or past n scans nothing and
  // its loads read nothing), so every path between a set's loads and their
  // use issues the other set's loads: the compiler's wait before a step
  // leaves the other step's loads in flight instead of draining them all.
  for (int s = 0; s < nsteps; s += 2) {
    int mark = tail;
    fair_share_priority(wslot);
    scan_step(sA, s);
    scan_issue(sA, s + 2);
    refine_until(mark);
    mark = tail;
    fair_share_priority(wslot);
    scan_step(sB, s + 1);
    scan_issue(sB, s + 3);
    refine_until(mark);
  }
  refine_until(tail);

  // ---- one partial per query head ----
  float l_h[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) l_h[tt] = group_sum<16>(lh[tt]);
  const size_t prow0 = hq0 * a.nc + c;   // partial row of head 0; heads are nc rows apart
  // head h's maximum and l sit in quad h % 4 of head tile h / 4; lane h
  // writes them
  float M = kNegInf, l = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float Mh = lane_value(mh[h >> 2], 16 * (h & 3));
    const float lhh = lane_value(l_h[h >> 2], 16 * (h & 3));
    M = lane == h ? Mh : M;
    l = lane == h ? lhh : l;
  }
  if (lane < G)
    *reinterpret_cast<f32x2*>(a.ml_part + (prow0 + (size_t)lane * a.nc) * 2) =
        f32x2{M == kNegInf ? kNegInf : M * cl2, l};
  // O rows through the V tiles (free now) so that every store writes 16
  // bytes per lane: rows h = 4 qg + e (h < G), dims 16 db + n16
  float* ost = reinterpret_cast<float*>(lv0);
  if (qg < NT) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) ost[(4 * qg + e) * D + 16 * db + n16] = o[db][e];
  }
#pragma unroll
  for (int i = 0; i < G * D / 4 / kWave; ++i) {
    const int f = i * kWave + lane;   // 16-byte piece f of G rows of D floats
    const int h = f / (D / 4), col = f % (D / 4);
    *reinterpret_cast<f32x4*>(a.o_part + (prow0 + (size_t)h * a.nc) * D + 4 * col) =
        *reinterpret_cast<const f32x4*>(ost + h * D + 4 * col);
  }
}

hipError_t launch_ffd_wave(int G, const FfdArgs& a, hipStream_t s) {
  const size_t units = (size_t)a.B * a.Hkv * a.nc;
  const dim3 grid((unsigned)((units + kWaves - 1) / kWaves)), block(kThreads);
  const bool mask = a.cand_mask != nullptr;
  if (G == 4 && mask) hipLaunchKernelGGL((ffd_wave_kernel<4, true>), grid, block, 0, s, a);
  else if (G == 4) hipLaunchKernelGGL((ffd_wave_kernel<4, false>), grid, block, 0, s, a);
  else if (G == 8 && mask) hipLaunchKernelGGL((ffd_wave_kernel<8, true>), grid, block, 0, s, a);
  else if (G == 8) hipLaunchKernelGGL((ffd_wave_kernel<8, false>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fdk
