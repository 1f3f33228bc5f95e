// Multi-row decode with two query tiles (16 < R = G*M <= 32 query rows per
// kv-head) on a pair of waves ("Flash Decoding" explainer, section 1; the
// flat GEMM case of the "FlashDecoding" deployment blog, section 1).
//
// A workgroup is two waves working on the same unit (sequence, kv-head,
// chunk).  Wave w owns query rows 16 w .. 16 w + 15, so each holds one
// query tile's accumulators instead of one wave holding both tiles.  A batch
// is eight 16-position tiles (128 positions) and a wave has the SIMD to
// itself, so its registers hold its four K and four V tiles in flight.  The
// K and V rows of a batch are read from HBM once: each wave loads half of
// the batch's tiles (tiles w, w + 2, w + 4, w + 6) with coalesced 16-byte
// loads and writes them into the workgroup's LDS, where both waves read
// every tile:
//
//   barrier 1   both waves are done reading the previous batch's tiles
//   own tiles   registers -> LDS, then the next batch's loads are issued
//   barrier 2   the batch is complete in LDS
//   compute     S^T = K Q^T per tile (v_mfma_f32_16x16x32_bf16, K rows the
//               A operand), online softmax per query row, P V over pairs of
//               tiles with 16x16x32 (V read back transposed with
//               ds_read_b64_tr_b16), p split into bf16 hi + lo parts
//
// The operand layouts and the softmax are those of the one-tile kernel
// (multirow.hpp).  At the end of a unit each wave stages its 16 O rows in
// its own two K tiles (after a barrier) so that every partial store writes
// 16 bytes per lane and whole rows; the stores go out beside the next
// batch's loads.
#include "multirow.hpp"

namespace fdk {

namespace {

constexpr int kPairTiles = 8;   // 16-position tiles per batch (four per wave)
// paged: pages per split at most (the page-id buffer); twice the one-tile
// kernel's, so that a worker of a ragged cache ends fewer units
constexpr int kPairPagePids = 2 * kMultiPagePids;

// LDS row strides (bytes) of the 16-row K and V tiles.  Row r of a K tile
// starts 4 r banks (of 4 bytes) on, so the 16-byte operand reads of rows
// 0-15 by a 16-lane group touch each bank once; row r of a V tile starts
// 8 r banks on, so the transposing 8-byte reads (rows 4 qd + n / 4, four
// 8-byte pieces each) of 32 lanes never share a bank (the same holds with 32
// banks).  The one-tile kernel's 8-byte padding (2 banks per row) gives 2x
// conflicts on the K and 4x on the V reads by that model; measured here:
// conflict cycles per LDS instruction 2.9 -> 0.95, M = 8 179.2 -> 176.8 us
// per call.  (The one-tile kernel measured 5 % slower with these strides
// and keeps its padding.)
template <int D>
constexpr int kKStride = 2 * D + 16;
template <int D>
constexpr int kVStride = 2 * D + 32;

// PAGED: k and v are page pools, as in the one-tile kernel.
template <int D, bool PAGED>
__global__ __launch_bounds__(2 * kWave) __attribute__((amdgpu_waves_per_eu(1)))
void multi_pair_kernel(MultiArgs a0) {
  // paged: the split may grow on the device (paged_split_factor)
  MultiArgs a = a0;
  constexpr int KS = D / 32;             // QK k-steps (32 dims each)
  constexpr int DB = D / 16;             // 16-dim blocks of the P V product
  constexpr int TT = kPairTiles;
  constexpr int TW = TT / 2;             // tiles of K and of V each wave loads
  constexpr int STEP = 16 * TT;          // positions per batch
  constexpr int ROWB = D * 2;            // bytes per cache row
  constexpr int LPR = ROWB / 16;         // lanes per row in a coalesced load
  constexpr int RPI = kWave / LPR;       // rows per wave load
  constexpr int NI = 16 / RPI;           // wave loads per 16-row tile
  constexpr int KSTR = kKStride<D>;      // LDS row strides of the K and V tiles
  constexpr int VSTR = kVStride<D>;
  constexpr int OSTR = D * 4 + 16;       // fp32 O row stride of the store staging
  constexpr int ORPI = kWave * 16 / (D * 4);   // O rows per wave store
  constexpr int LPO = kWave / ORPI;            // lanes per O row
  static_assert(8 * OSTR <= 16 * KSTR, "eight O rows must fit one K tile");
  __shared__ __align__(16) unsigned char s_k[TT][16 * KSTR];
  __shared__ __align__(16) unsigned char s_v[TT][16 * VSTR];
  // paged: each wave's copy of the page ids of the current and next split
  __shared__ int s_pid[PAGED ? 2 : 1][2][PAGED ? kPairPagePids : 1];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, qd = lane >> 4;
  const int G = a.Hq / a.Hkv, R = G * a.M;
  const int n_units = a.B * a.Hkv * a.nc;
  const int row0 = 16 * wave;            // this wave's first query row
  const int lrow = lane / LPR, lcol = lane % LPR;
  const int lane_off = lrow * ROWB + 16 * lcol;
  // transposing read of a V tile: lane (n, qd) gets V[4 qd + e][16 db + n]
  const int tr_off = (4 * qd + (n >> 2)) * VSTR + 8 * (n & 3);
  const float c_log2 = a.c_log2;

  // a unit: sequence b (holding L positions), kv-head, split c = [c0, c1)
  // (empty when a paged sequence is shorter than the split's start)
  struct UnitM {
    int b, kvh, c, c0, c1, L, xw;
  };
  auto seq_len = [&](int b) {
    if constexpr (PAGED) {
      const auto* sl = (const __attribute__((address_space(4))) int32_t*)a.seq_lens;
      return min(max(sl[__builtin_amdgcn_readfirstlane(b)], 0), a.L);
    } else {
      return a.L;
    }
  };
  PagedWalk walk{};   // paged: the units that hold positions
  // paged: this workgroup's units [u_first, u_last], the first from
  // position pos0, the last up to pos1 (paged_worker_range)
  int u_first = -1, u_last = -1, pos0 = 0, pos1 = 0;
  auto decode = [&](int u, UnitM& x) {
    if constexpr (PAGED) {
      paged_walk_decode(a, u, walk, x.b, x.kvh, x.c);
    } else {
      x.c = u % a.nc;
      const int bk = u / a.nc;
      x.kvh = bk % a.Hkv;
      x.b = bk / a.Hkv;
    }
    x.L = seq_len(x.b);
    x.c0 = x.c * a.chunk;
    x.c1 = min(x.c0 + a.chunk, x.L);
    x.xw = -1;
    if constexpr (PAGED) {
      if (u == u_first && x.c0 < pos0) {
        x.c0 = pos0;
        x.xw = (int)blockIdx.x;
      }
      if (u == u_last) x.c1 = min(x.c1, pos1);
    }
  };
  // paged: the pool page of each of this wave's tiles of the batch at T
  // (uniform; 0 for tiles past the chunk end c1, which read nothing).  Read
  // from LDS before the batch's tiles are written there, so that waiting
  // for these reads does not also wait for those writes.
  const int shift = a.page_shift, pmask = (1 << a.page_shift) - 1;
  auto tile_pages = [&](const UnitM& x, int buf, int T, int c1, int (&pg)[TW]) {
    if constexpr (PAGED) {
#pragma unroll
      for (int j = 0; j < TW; ++j) {
        const int t0 = T + 16 * (2 * j + wave);
        const int p = t0 < c1 ? s_pid[wave][buf][(t0 - x.c0) >> shift] : 0;
        pg[j] = min(max(__builtin_amdgcn_readfirstlane(p), 0), a.num_pages - 1);
      }
    }
  };
  // first byte of row t0 (a multiple of 16) of unit x's K or V; pg: its
  // pool page (paged)
  auto row_base = [&](const void* t, const UnitM& x, int pg, int t0) {
    if constexpr (PAGED) {
      return reinterpret_cast<const char*>(t) +
             ((((size_t)pg * a.Hkv + x.kvh) << shift) + (size_t)(t0 & pmask)) * ROWB;
    } else {
      return reinterpret_cast<const char*>(t) +
             (((size_t)x.b * a.Hkv + x.kvh) * (size_t)a.L + (size_t)t0) * ROWB;
    }
  };
  // query row row0 + n: token r = row / G, head kvh*G + row % G, last
  // visible position L - M + r; rows >= R are padding (q = 0)
  const int qrow = row0 + n;
  u32x4 qf[KS];
  auto load_q = [&](const UnitM& x) {
    if (qrow < R) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                           (((size_t)x.b * a.M + qrow / G) * a.Hq + (size_t)x.kvh * G + qrow % G) * D +
                           8 * qd;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = ld16(qp + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = u32x4{0, 0, 0, 0};
    }
  };
  // this wave's tiles 2 j + wave of the batch at T (pages pg, tile_pages):
  // one buffer descriptor per tile, limited to the chunk end c1 (rows past
  // it read as zeros, untouched)
  auto issue = [&](const void* t, const UnitM& x, const int (&pg)[TW], int T, int c1,
                   u32x4 (&r)[TW][NI]) {
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int t0 = T + 16 * (2 * j + wave);
      const int nrow = min(max(c1 - t0, 0), 16);
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(row_base(t, x, pg[j], t0), nrow * ROWB);
#pragma unroll
      for (int i = 0; i < NI; ++i) r[j][i] = ld16_buf(rs, lane_off + RPI * i * ROWB);
    }
  };
  auto to_lds = [&](unsigned char* dst, const u32x4 (&r)[NI], int str) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<u32x4*>(dst + (RPI * i + lrow) * str + 16 * lcol) = r[i];
  };
  // O rows 0-7 of this wave staged in K tile `wave`, rows 8-15 in K tile
  // wave + 2 (tiles that only this wave writes)
  auto o_stage = [&](int r) { return s_k[wave + 2 * (r >> 3)] + (r & 7) * OSTR; };

  // partials of unit x: rows ((b*M + r)*Hq + h)*nc + c; called after a
  // barrier, when no wave reads the tiles any more
  // (x as decoded when the unit ran: the paged walker only moves forward)
  // partial row of query row r (< R) of unit x, in o_part / ml_part or, for
  // a part cut off a split's start, in x_o / x_ml
  auto part_row = [&](const UnitM& x, int r) {
    return x.xw >= 0 ? (size_t)x.xw * R + r
                     : (((size_t)x.b * a.M + r / G) * a.Hq + (size_t)x.kvh * G + r % G) * a.nc +
                           x.c;
  };
  // A finished unit's partials are staged into registers (through the
  // wave's own two K tiles, for 16-byte stores of whole rows) and written,
  // non-temporally (the merge reads them once, in another launch), after
  // the next batch's loads are issued: stores and loads share one wait
  // counter, and beside the next loads their latency overlaps theirs.
  constexpr int NST = 16 / ORPI;   // 16-byte stores per lane per unit
  f32x4 pv[NST];
  f32x2 pml = f32x2{0.f, 0.f};
  UnitM px{};
  bool pend = false;   // wave-uniform
  auto stage_unit = [&](const f32x4 (&o)[DB], float m, float l, const UnitM& x) {
    pml = f32x2{(m == kNegInf) ? kNegInf : m * c_log2, l};
    // lane (n, qd) holds O rows 4 qd + e, dims 16 db + n
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float*>(o_stage(4 * qd + e) + (16 * db + n) * 4) = o[db][e];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int rr = ORPI * i + lane / LPO, cb = 16 * (lane % LPO);
      pv[i] = *reinterpret_cast<const f32x4*>(o_stage(rr) + cb);
    }
    px = x;
    pend = true;
  };
  auto flush = [&]() {
    if (!pend) return;
    pend = false;
    float* const op = px.xw >= 0 ? a.x_o : a.o_part;
    float* const mlp = px.xw >= 0 ? a.x_ml : a.ml_part;
    if (qd == 0 && qrow < R)
      __builtin_nontemporal_store(pml, reinterpret_cast<f32x2*>(mlp + part_row(px, qrow) * 2));
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int rr = ORPI * i + lane / LPO, cb = 16 * (lane % LPO);
      const int row = row0 + rr;
      if (row < R)
        __builtin_nontemporal_store(
            pv[i], reinterpret_cast<f32x4*>(reinterpret_cast<unsigned char*>(op + part_row(px, row) * D) +
                                            cb));
    }
  };

  // workgroup w takes the consecutive units [w*per, (w+1)*per) (paged: the
  // units of its range of pages, paged_worker_range; both waves compute
  // the same range)
  int u, u_end;
  if constexpr (PAGED) {
    const long long P = paged_pages(a, lane);
    const int F = paged_split_factor(a, P, (int)gridDim.x, kPairPagePids);
    a.chunk *= F;
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.x_split = F;   // for the merge
    PagedSpot s0{}, s1{};
    const bool any =
        paged_worker_range(a, lane, (int)blockIdx.x, (int)gridDim.x, P, s0, s1);
    if ((int)blockIdx.x < a.x_cap && threadIdx.x == 0) {
      int32_t* mt = a.x_meta + 4 * (size_t)blockIdx.x;
      mt[0] = s0.b;
      mt[1] = s0.kvh;
      mt[2] = s0.c;
      mt[3] = any && s0.pos % a.chunk != 0 ? 1 : 0;
    }
    if (!any) return;   // both waves of the workgroup
    u = __builtin_amdgcn_readfirstlane(s0.u);
    u_end = __builtin_amdgcn_readfirstlane(s1.u) + 1;
    u_first = u;
    u_last = u_end - 1;
    pos0 = __builtin_amdgcn_readfirstlane(s0.pos);
    pos1 = __builtin_amdgcn_readfirstlane(s1.pos) + (1 << a.page_shift);
    walk.b = __builtin_amdgcn_readfirstlane(s0.b);
    walk.first = __builtin_amdgcn_readfirstlane(s0.first);
    walk.units = __builtin_amdgcn_readfirstlane(s0.units);
  } else {
    const int per = (n_units + (int)gridDim.x - 1) / (int)gridDim.x;
    u = (int)blockIdx.x * per;
    u_end = min(u + per, n_units);
    if (u >= n_units) return;   // both waves of the workgroup
  }
  UnitM cur;
  decode(u, cur);
  u32x4 kr[TW][NI], vr[TW][NI];
  int buf = 0;   // LDS copy of the current unit's page ids (paged)
  int pid[kPairPagePids / kWave];
  if constexpr (PAGED) {
    page_ids_load<kPairPagePids>(a, cur.b, cur.c0, cur.c1, lane, pid);
    page_ids_store<kPairPagePids>(s_pid[wave][0], lane, pid);
  }
  load_q(cur);
  int pg[TW] = {};
  tile_pages(cur, buf, cur.c0, cur.c1, pg);
  issue(a.k, cur, pg, cur.c0, cur.c1, kr);
  issue(a.v, cur, pg, cur.c0, cur.c1, vr);
  while (true) {
    const int un = u + 1;
    const bool has_next = un < u_end;
    UnitM nxt = cur;
    if (has_next) decode(un, nxt);
    if constexpr (PAGED) {
      if (has_next) page_ids_load<kPairPagePids>(a, nxt.b, nxt.c0, nxt.c1, lane, pid);
    }
    const int c0 = cur.c0, c1 = cur.c1;
    const int lim = cur.L - a.M + qrow / G;

    f32x4 o[DB];
    float m = kNegInf, l = 0.f;   // row's running maximum (raw), this lane's part of l
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int T = c0; T < c1; T += STEP) {
      __syncthreads();   // the previous batch's tiles are read
      // next batch's loads, the next unit's first after the last batch; one
      // issue path (scalar selects), so that the compiler's wait counts
      // agree on every path.  After the wave's last batch the limit is 0:
      // the loads return zeros without touching memory.
      const bool last = T + STEP >= c1;
      UnitM xs = cur;
      int t_next = T + STEP, c_end = c1, b_next = buf;
      if (last) {
        if constexpr (PAGED) {
          if (has_next) page_ids_store<kPairPagePids>(s_pid[wave][buf ^ 1], lane, pid);
        }
        xs = nxt;
        b_next = buf ^ 1;
        t_next = has_next ? nxt.c0 : T;
        c_end = has_next ? nxt.c1 : T;
      }
      tile_pages(xs, b_next, t_next, c_end, pg);
#pragma unroll
      for (int j = 0; j < TW; ++j) {
        to_lds(s_k[2 * j + wave], kr[j], KSTR);
        to_lds(s_v[2 * j + wave], vr[j], VSTR);
      }
      issue(a.k, xs, pg, t_next, c_end, kr);
      issue(a.v, xs, pg, t_next, c_end, vr);
      flush();   // the previous unit's partials
      __syncthreads();   // the batch is in LDS

      float sc[TT][4];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        // A operand of k-step s: dims 32 s + 8 qd .. +8 of K row n
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(s_k[tt] + n * KSTR + 64 * s + 16 * qd);
          acc = mfma_qk(ka, qf[s], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = T + 16 * tt + 4 * qd + e;
          sc[tt][e] = (pos < c1 && pos <= lim) ? acc[e] : kNegInf;
        }
      }
      // the query of the next unit (qf is no longer needed for this one)
      if (last && has_next) load_q(nxt);

      float bm = kNegInf;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) bm = fmaxf(bm, sc[tt][e]);
      bm = pair_max<32>(pair_max<16>(bm));
      const float mn = fmaxf(m, bm);
      if (__any(mn > m)) {
        const float alpha = (mn == m) ? 1.f : exp2_hw((m - mn) * c_log2);
        l *= alpha;
        // O rows 4*qd + e take the factors of those rows (held by lanes 4*qd + e)
        float ae[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ae[e] = __shfl(alpha, 4 * qd + e);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][e] *= ae[e];
        m = mn;
      }
      // exponent (s - m) c: exactly 0 at the running maximum
      const float base = (m == kNegInf) ? 0.f : m;
      u32x2 ph[TT], pl[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = exp2_hw((sc[tt][e] - base) * c_log2);
          l += p[e];
        }
        split_bf16(p, ph[tt], pl[tt]);
      }
      // P V over pairs of tiles: k = 8 qd + j stands for position 4 qd + j % 4
      // of tile 2 tp + j / 4
#pragma unroll
      for (int tp = 0; tp < TT / 2; ++tp) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 v0 = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                         (__attribute__((address_space(3))) s16x4_t*)(s_v[2 * tp] + tr_off + 32 * db)));
          const u32x2 v1 = __builtin_bit_cast(
              u32x2,
              __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) s16x4_t*)(s_v[2 * tp + 1] + tr_off + 32 * db)));
          const u32x4 vv = u32x4{v0.x, v0.y, v1.x, v1.y};
          const u32x2 h0 = ph[2 * tp], h1 = ph[2 * tp + 1];
          const u32x2 l0 = pl[2 * tp], l1 = pl[2 * tp + 1];
          o[db] = mfma_qk(u32x4{h0.x, h0.y, h1.x, h1.y}, vv, o[db]);
          o[db] = mfma_qk(u32x4{l0.x, l0.y, l1.x, l1.y}, vv, o[db]);
        }
      }
    }
    // l of row n: the four lanes of the row hold parts
    l = pair_sum<32>(pair_sum<16>(l));
    __syncthreads();   // no wave reads the tiles any more
    flush();   // still pending only when this unit ran no batch
    stage_unit(o, m, l, cur);
    if constexpr (PAGED) {
      // an empty split ran no batch, so nothing requested the next one's
      // query and first rows yet
      if (c1 <= c0 && has_next) {
        load_q(nxt);
        page_ids_store<kPairPagePids>(s_pid[wave][buf ^ 1], lane, pid);
        tile_pages(nxt, buf ^ 1, nxt.c0, nxt.c1, pg);
        issue(a.k, nxt, pg, nxt.c0, nxt.c1, kr);
        issue(a.v, nxt, pg, nxt.c0, nxt.c1, vr);
      }
    }
    if (!has_next) break;
    cur = nxt;
    u = un;
    if constexpr (PAGED) buf ^= 1;
  }
  flush();
}

// Units that run at once: one per workgroup (wave pair).
template <int D>
size_t pair_slots() {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, multi_pair_kernel<D, false>, 2 * kWave,
                                                     0) !=
            hipSuccess ||
        nb <= 0)
      nb = 1;
    return nb;
  }();
  return (size_t)cu_count() * per_cu;
}

// *workers: the workgroups launched (each a worker of a paged call).
template <int D>
hipError_t launch_pair(const MultiArgs& a, hipStream_t s, int* workers) {
  auto kernel = a.block_table != nullptr ? multi_pair_kernel<D, true> : multi_pair_kernel<D, false>;
  // equal rounds for every workgroup
  const size_t units = (size_t)a.B * a.Hkv * a.nc;
  const size_t slots = pair_slots<D>();
  const size_t rounds = (units + slots - 1) / slots;
  // paged: every resident workgroup (the pages are divided over the workers)
  const unsigned grid = a.block_table != nullptr ? (unsigned)std::min(units, slots)
                                                 : (unsigned)((units + rounds - 1) / rounds);
  *workers = (int)grid;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(2 * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t multi_pair_slots(int D) { return D == 64 ? pair_slots<64>() : pair_slots<128>(); }

hipError_t launch_multi_pair(int D, const MultiArgs& a, hipStream_t s, int* workers) {
  if (D == 64) return launch_pair<64>(a, s, workers);
  if (D == 128) return launch_pair<128>(a, s, workers);
  return hipErrorInvalidValue;
}

}  // namespace fdk
