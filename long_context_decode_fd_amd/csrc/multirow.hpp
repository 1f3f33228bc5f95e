// Multi-row decode attention for gfx950: M new query tokens per sequence,
// each attending to the cache up to its own position ("Flash Decoding"
// explainer, section 1; the tokens' keys and values are already appended at
// positions L-M .. L-1).  The G query heads of a kv-head times the M tokens
// give R = G*M query rows that share every K and V row -- the flat GEMM case
// of the "FlashDecoding" deployment blog (section 1), which here runs on the
// matrix cores.  This kernel takes R <= 16 rows (one query tile) per wave;
// 16 < R <= 32 runs on a pair of waves (multirow_pair.hip) with the same
// operand layouts:
//
//   * K and V rows arrive with fully coalesced 16-byte loads (one wave load
//     = 1 KiB of consecutive rows) and pass through a small per-wave LDS
//     tile, from which each lane reads its MFMA operand.
//   * S^T = K Q^T per 16-position tile with v_mfma_f32_16x16x32_bf16: the A
//     operand is 16 K rows (lane (n, quad) holds dims 32s + 8 quad .. +8 of
//     row n at k-step s), the B operand the query rows (same lane map).  In
//     the 16x16 result a lane holds one query row n and four consecutive
//     positions 4*quad .. 4*quad+3, which is exactly the A operand layout of
//     v_mfma_f32_16x16x16_bf16 for P V.
//   * Online softmax per query row over the wave's batch (row maximum across
//     the four lanes of the row with two shuffles); p in fp32, split into
//     bf16 hi + lo parts so that P V keeps fp32-level accuracy (two MFMAs).
//   * V tiles are read back from LDS transposed with ds_read_b64_tr_b16 (four
//     positions of one dim per lane, the B operand of P V).
//   * Split-KV as in the single-query kernel: one wavefront per split,
//     partials (O, m, l) per (token, head, split), merged by the common exact
//     log-sum-exp kernel.
#pragma once

#include <algorithm>

#include "internal.hpp"
#include "splitkv.hpp"

namespace fdk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// 16-position tiles per wave batch: 2 K and 2 V tiles in flight (8 + 8
// wave loads at d = 128)
constexpr int kMrTiles = 2;
// finished units held in registers before their partials are written
constexpr int kMrHold = 4;

__device__ __forceinline__ f32x4 mfma_qk(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_pv(const u32x2& a, const u32x2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                    __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// p = hi + lo with hi = bf16(p), lo = bf16(p - hi), both rounded to nearest
// even by the hardware conversion (two values per instruction): two bf16
// pairs from four fp32 values.
__device__ __forceinline__ void split_bf16(const float (&p)[4], u32x2& hi, u32x2& lo) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float a = p[2 * j], b = p[2 * j + 1];
    h[j] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)a, (__bf16)b});
    const float ra = a - __uint_as_float(h[j] << 16);
    const float rb = b - __uint_as_float(h[j] & 0xFFFF0000u);
    l[j] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)ra, (__bf16)rb});
  }
  hi = u32x2{h[0], h[1]};
  lo = u32x2{l[0], l[1]};
}

// Paged caches: the block-table entries of a split [c0, c1) of sequence b,
// kMultiPagePids / 64 per lane, read into registers first and written to
// the wave's LDS copy later, as read: any arithmetic on them here would let
// the compiler move it (and a wait for every load in flight) up to the
// loads; they are clamped to [0, num_pages) where a tile reads them.
constexpr int kPidPerLane = kMultiPagePids / kWave;

// Every lane loads (entries past the split repeat its last page), so that no
// register is written but by a load: a default value written into a
// register whose previous load may still be in flight would make the
// compiler wait for every load issued before it.  A split holds positions
// (c0 < c1 <= the sequence's length), so its entries lie inside the table row.
template <int NP = kMultiPagePids>
__device__ __forceinline__ void page_ids_load(const MultiArgs& a, int b, int c0, int c1,
                                              int lane, int (&v)[NP / kWave]) {
  const int shift = a.page_shift;
  const int last = max((c1 - c0 + (1 << shift) - 1) >> shift, 1) - 1;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages + (c0 >> shift);
#pragma unroll
  for (int j = 0; j < NP / kWave; ++j) v[j] = bt[min(lane + j * kWave, last)];
}

template <int NP = kMultiPagePids>
__device__ __forceinline__ void page_ids_store(int* dst, int lane, const int (&v)[NP / kWave]) {
#pragma unroll
  for (int j = 0; j < NP / kWave; ++j) dst[lane + j * kWave] = v[j];
}

// Paged caches: the units that hold positions, (b, kvh, c) with
// c < ceil(L_b / chunk), numbered sequence after sequence, kv-head-major
// inside a sequence, so that a wave's consecutive units are consecutive
// chunks of one (sequence, kv-head) and no wave waits on empty ones.  The
// walker's state is wave-uniform; lengths come through the scalar cache
// (their wait is on the scalar counter, not on the vector-memory counter of
// the K and V loads in flight).
struct PagedWalk {
  int b, first, units;   // sequence b's units are [first, first + units)
};

__device__ __forceinline__ int paged_len_u(const MultiArgs& a, int b) {
  const auto* sl = (const __attribute__((address_space(4))) int32_t*)a.seq_lens;
  return min(max(sl[__builtin_amdgcn_readfirstlane(b)], 0), a.L);
}

// units of sequence b (b < B)
__device__ __forceinline__ int paged_units_u(const MultiArgs& a, int b) {
  return a.Hkv * ((paged_len_u(a, b) + a.chunk - 1) / a.chunk);
}

// Units of the whole call, and the walker positioned at the sequence that
// holds unit u (u below the total; else at the end): 64 sequences per step,
// an inclusive scan across the lanes, the first lane whose running total
// passes u.
__device__ __forceinline__ int paged_walk_start(const MultiArgs& a, int lane, int u,
                                                PagedWalk& w) {
  int first = 0, found = 0;
  w.b = a.B;
  w.first = 0;
  w.units = 0;
  for (int base = 0; base < a.B; base += kWave) {   // wave-uniform
    const int bb = base + lane;
    const int mine = bb < a.B
                         ? a.Hkv * ((min(max(a.seq_lens[bb], 0), a.L) + a.chunk - 1) / a.chunk)
                         : 0;
    int incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
    if (!found && u < first + total) {
      const uint64_t past = __builtin_amdgcn_ballot_w64(first + incl > u);
      const int l = (int)__builtin_ctzll(past);
      w.b = base + l;
      w.units = __builtin_amdgcn_readlane(mine, l);
      w.first = first + __builtin_amdgcn_readlane(incl, l) - w.units;
      found = 1;
    }
    first += total;
  }
  return first;
}

// A worker's share of a paged call.  The call's pages are counted in unit
// order (sequence after sequence, kv-head-major inside a sequence: a
// (sequence, kv-head) holds ceil(L_b / page) of them) and split evenly:
// worker w of n' takes pages [w P / n', (w + 1) P / n'), with n' = min(n,
// x_cap, P / pages-per-split), so every range spans at least a split's
// pages and a split is cut at most once.  Whole units would leave workers
// idle or a whole unit apart (7,224 units of 1,024 positions over 1,016
// waves: 903 waves with 8 units, 113 with none).  The range's units run
// from the one holding its first page (from that page's position on: a
// part cut off the split's start) to the one holding its last page (up to
// that page's end).
struct PagedSpot {
  int u;                 // unit holding the page
  int pos;               // the page's first position in its (sequence, kv-head)
  int b, kvh, c;         // that unit
  int first, units;      // sequence b's units are [first, first + units)
};

// a wave-uniform 64-bit value into scalar registers
__device__ __forceinline__ long long uniform_ll(long long x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ long long scan_incl_ll(long long x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long t = __shfl_up(x, o);
    if (lane >= o) x += t;
  }
  return x;
}

// Pages of the call (wave-uniform).
__device__ __forceinline__ long long paged_pages(const MultiArgs& a, int lane) {
  const int shift = a.page_shift;
  long long P = 0;
  for (int base = 0; base < a.B; base += kWave) {   // wave-uniform
    const int bb = base + lane;
    const int Lb = bb < a.B ? min(max(a.seq_lens[bb], 0), a.L) : 0;
    const long long npb = (Lb + (1 << shift) - 1) >> shift;
    P += uniform_ll(__shfl(scan_incl_ll((long long)a.Hkv * npb, lane), kWave - 1));
  }
  return P;
}

// Workers that take part: n, at most x_cap, and few enough that each range
// spans a split's pages (at least one while there are pages).
__device__ __forceinline__ long long paged_workers(const MultiArgs& a, long long P, int n) {
  const int cpp = a.chunk >> a.page_shift;   // pages per split (a multiple of the page)
  return P > 0 ? max(min((long long)min(n, a.x_cap), P / cpp), 1LL) : 0;
}

// Split factor F: the split grows to chunk * F (F a power of two, at most
// 256, and at most max_pages pages: the kernel's page-id buffer) while the
// same number of workers still get a split's pages each.  Longer splits cut
// the partials written and merged and the unit changes; the workers' count
// keeps the device busy (the lengths decide it, so it is chosen here, not
// by the host).
__device__ __forceinline__ int paged_split_factor(const MultiArgs& a, long long P, int n,
                                                  int max_pages = kMultiPagePids) {
  const int cpp = a.chunk >> a.page_shift;
  const long long na = paged_workers(a, P, n);
  int F = 1;
  while (2 * F <= 256 && cpp * 2 * F <= max_pages && P / ((long long)cpp * 2 * F) >= na) F *= 2;
  return F;
}

// false: worker w has no pages.  Else s0 / s1 locate its first / last page.
// P: paged_pages(a).
__device__ __forceinline__ bool paged_worker_range(const MultiArgs& a, int lane, int w, int n,
                                                   long long P, PagedSpot& s0, PagedSpot& s1) {
  const int shift = a.page_shift, page = 1 << shift;
  const int cpp = a.chunk >> shift;   // pages per split (the split is a multiple of the page)
  auto lens = [&](int bb, int& Lb, int& npb, int& nsb) {
    Lb = bb < a.B ? min(max(a.seq_lens[bb], 0), a.L) : 0;
    npb = (Lb + page - 1) >> shift;
    nsb = (Lb + a.chunk - 1) / a.chunk;
  };
  const long long na = paged_workers(a, P, n);
  if (w >= na) return false;
  const long long g0 = (long long)w * P / na, g1 = (long long)(w + 1) * P / na - 1;
  long long fp = 0;
  int fu = 0;
  bool f0 = false, f1 = false;
  for (int base = 0; base < a.B && !(f0 && f1); base += kWave) {   // wave-uniform
    int Lb, npb, nsb;
    lens(base + lane, Lb, npb, nsb);
    const long long ip = scan_incl_ll((long long)a.Hkv * npb, lane);
    int iu = a.Hkv * nsb;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(iu, o);
      if (lane >= o) iu += t;
    }
    const long long totp = uniform_ll(__shfl(ip, kWave - 1));
    const int totu = __builtin_amdgcn_readfirstlane(__shfl(iu, kWave - 1));
    auto locate = [&](long long g, PagedSpot& sp) {
      const int l = __builtin_amdgcn_readfirstlane(
          (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(fp + ip > g)));
      const int npl = __shfl(npb, l), nsl = __shfl(nsb, l);
      const int npu = __builtin_amdgcn_readfirstlane(npl), nsu = __builtin_amdgcn_readfirstlane(nsl);
      const long long pstart = fp + uniform_ll(__shfl(ip, l)) - (long long)a.Hkv * npu;
      const int off = (int)(g - pstart);
      sp.b = base + l;
      sp.units = a.Hkv * nsu;
      sp.first = __builtin_amdgcn_readfirstlane(fu + __shfl(iu, l)) - sp.units;
      sp.kvh = off / npu;
      const int p = off - sp.kvh * npu;
      sp.c = p / cpp;
      sp.pos = p << shift;
      sp.u = sp.first + sp.kvh * nsu + sp.c;
    };
    if (!f0 && g0 < fp + totp) {
      locate(g0, s0);
      f0 = true;
    }
    if (!f1 && g1 < fp + totp) {
      locate(g1, s1);
      f1 = true;
    }
    fp += totp;
    fu += totu;
  }
  return true;
}

// (b, kvh, c) of unit u; u must not decrease from call to call
__device__ __forceinline__ void paged_walk_decode(const MultiArgs& a, int u, PagedWalk& w,
                                                  int& b, int& kvh, int& c) {
  while (u >= w.first + w.units) {   // wave-uniform
    w.first += w.units;
    ++w.b;
    w.units = paged_units_u(a, w.b);
  }
  b = w.b;
  const int ns = w.units / a.Hkv;
  const int r = u - w.first;
  kvh = r / ns;
  c = r - kvh * ns;
}

// One query tile of R = G*M <= 16 rows per wave.  PAGED: k and v are page
// pools (MultiArgs), each 16-row tile lies in one page (pages of 16 rows or
// more, tiles aligned to 16).
template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void multi_kernel(MultiArgs a0) {
  // paged: the split may grow on the device (paged_split_factor)
  MultiArgs a = a0;
  constexpr int KS = D / 32;             // QK k-steps (32 dims each)
  constexpr int DB = D / 16;             // 16-dim blocks of the P V product
  constexpr int TT = kMrTiles;
  constexpr int STEP = 16 * TT;          // positions per wave batch
  constexpr int ROWB = D * 2;            // bytes per cache row
  constexpr int LPR = ROWB / 16;         // lanes per row in a coalesced load
  constexpr int RPI = kWave / LPR;       // rows per wave load
  constexpr int NI = 16 / RPI;           // wave loads per 16-row tile (= KS)
  constexpr int LSTR = ROWB + 8;         // LDS row stride: rows 4 apart sit 8 banks apart
  constexpr int OSTR = D * 4 + 16;       // fp32 O row stride of the store staging
  constexpr int ORPI = kWave * 16 / (D * 4);   // O rows per wave store
  static_assert(16 * OSTR <= 2 * 16 * LSTR, "O staging must fit the wave's K/V tiles");
  __shared__ __align__(16) unsigned char s_kv[kWaves][2][16 * LSTR];
  // paged: page ids of the wave's current and next split
  __shared__ int s_pid[PAGED ? kWaves : 1][2][PAGED ? kMultiPagePids : 1];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, qd = lane >> 4;
  const int G = a.Hq / a.Hkv, R = G * a.M;
  const int stride = (int)gridDim.x * kWaves;
  const int n_units = a.B * a.Hkv * a.nc;
  unsigned char* lk = s_kv[wave][0];
  unsigned char* lv = s_kv[wave][1];
  const int lrow = lane / LPR, lcol = lane % LPR;   // coalesced-load lane map
  // Transposing LDS read (ds_read_b64_tr_b16): in each 16-lane group, lane i
  // receives element i % 4 of the 8-byte reads of lanes i/4, 4 + i/4, 8 + i/4
  // and 12 + i/4.  Lane n of quad qd therefore points at row 4*qd + n/4, dims
  // 16*db + 4*(n % 4) of the V tile, and gets V[4*qd + e][16*db + n], e < 4:
  // four positions of one dim, the B operand of P V.
  const int tr_off = (4 * qd + (n >> 2)) * LSTR + 8 * (n & 3);
  const float c_log2 = a.c_log2;

  // a unit: sequence b (holding L positions), kv-head, split c = [c0, c1)
  // (empty when a paged sequence is shorter than the split's start); xw >= 0:
  // a part cut off the split's start, whose partials go to worker slot xw
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
  const int wid = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kWaves + wave);
  PagedWalk walk{};   // paged: the units that hold positions
  // paged: this worker's units [u_first, u_last], the first from position
  // pos0, the last up to pos1
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
        x.xw = wid;
      }
      if (u == u_last) x.c1 = min(x.c1, pos1);
    }
  };
  // first byte of row t0 (a multiple of 16 in [c0, c1) when `used`; else
  // nothing is read there and any row will do) of unit x's K or V
  const int shift = a.page_shift, pmask = (1 << a.page_shift) - 1;
  auto row_base = [&](const void* t, const UnitM& x, int buf, int t0, bool used) {
    if constexpr (PAGED) {
      const int p = used ? s_pid[wave][buf][(t0 - x.c0) >> shift] : 0;
      const int pc = min(max(__builtin_amdgcn_readfirstlane(p), 0), a.num_pages - 1);
      return reinterpret_cast<const char*>(t) +
             ((((size_t)pc * a.Hkv + x.kvh) << shift) + (size_t)(t0 & pmask)) * ROWB;
    } else {
      return reinterpret_cast<const char*>(t) +
             (((size_t)x.b * a.Hkv + x.kvh) * (size_t)a.L + (size_t)t0) * ROWB;
    }
  };
  // Query row n of this lane: token r = n / G, head kvh*G + n % G; its last
  // visible position is L - M + r.  Rows >= R are padding (q = 0).
  u32x4 qf[KS];
  auto load_q = [&](const UnitM& x) {
    if (n < R) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                           (((size_t)x.b * a.M + n / G) * a.Hq + (size_t)x.kvh * G + n % G) * D +
                           8 * qd;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = ld16(qp + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = u32x4{0, 0, 0, 0};
    }
  };
  // wave load i of tile tt: rows T + 16*tt + RPI*i + lrow, bytes 16*lcol.
  // Buffer loads: each 16-row tile gets a descriptor whose base is the tile's
  // first row and whose byte limit ends at the chunk end c1, so every lane
  // uses the same offset (lrow, lcol) plus an immediate per load, with no
  // per-load address arithmetic; rows at or past c1 are outside the limit
  // and read as zeros without touching memory (their scores are masked and
  // their p is 0).  The range check covers the lane offset plus the
  // immediate; the scalar offset is 0.
  const int lane_off = lrow * ROWB + 16 * lcol;
  auto issue = [&](const void* t, const UnitM& x, int buf, int T, int c1,
                   u32x4 (&r)[TT][NI]) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t0 = T + 16 * tt;
      const int nrow = min(max(c1 - t0, 0), 16);
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(row_base(t, x, buf, t0, nrow > 0), nrow * ROWB);
#pragma unroll
      for (int i = 0; i < NI; ++i) r[tt][i] = ld16_buf(rs, lane_off + RPI * i * ROWB);
    }
  };
  // a tile of 16 rows into this wave's LDS tile (row-major, stride LSTR)
  auto to_lds = [&](unsigned char* dst, const u32x4 (&r)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<u32x4*>(dst + (RPI * i + lrow) * LSTR + 16 * lcol) = r[i];
  };

  // Partials of unit x, rows ((b*M + r)*Hq + h)*nc + c.  O goes through the
  // wave's LDS tiles (free between units: the next unit's K rows are still
  // in registers) so that every store writes 16 bytes per lane and whole
  // rows, instead of 4 bytes per lane in 64-byte pieces.
  unsigned char* ost = s_kv[wave][0];
  // (x as decoded when the unit ran: the paged walker only moves forward)
  // partial row of query row r (< R) of unit x, in o_part / ml_part or, for
  // a part cut off a split's start, in x_o / x_ml
  auto part_row = [&](const UnitM& x, int r) {
    return x.xw >= 0 ? (size_t)x.xw * R + r
                     : (((size_t)x.b * a.M + r / G) * a.Hq + (size_t)x.kvh * G + r % G) * a.nc +
                           x.c;
  };
  auto store_unit = [&](const f32x4 (&o)[DB], float m, float l, const UnitM& x) {
    float* const op = x.xw >= 0 ? a.x_o : a.o_part;
    float* const mlp = x.xw >= 0 ? a.x_ml : a.ml_part;
    if (qd == 0 && n < R)
      *reinterpret_cast<f32x2*>(mlp + part_row(x, n) * 2) =
          f32x2{(m == kNegInf) ? kNegInf : m * c_log2, l};
    // lane (n, qd) holds O rows 4*qd + e, dims 16*db + n
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float*>(ost + (4 * qd + e) * OSTR + (16 * db + n) * 4) = o[db][e];
    // read back: wave store i covers rows ORPI*i .. +ORPI, 16 bytes per lane
    constexpr int LPO = kWave / ORPI;   // lanes per O row
#pragma unroll
    for (int i = 0; i < 16 / ORPI; ++i) {
      const int row = ORPI * i + lane / LPO, cb = 16 * (lane % LPO);
      const f32x4 v = *reinterpret_cast<const f32x4*>(ost + row * OSTR + cb);
      if (row < R)
        *reinterpret_cast<f32x4*>(reinterpret_cast<unsigned char*>(op + part_row(x, row) * D) +
                                  cb) = v;
    }
  };
  // Finished units wait in registers (up to H of them) and are written
  // together when H are held or the wave has no unit left.  Stores count on
  // the same vector-memory counter as loads: partials stored between units
  // made the next unit's first K wait for them.
  constexpr int H = kMrHold;
  f32x4 hold_o[H][DB];
  float hold_m[H], hold_l[H];
  UnitM hold_x[H];
  int held = 0;   // wave-uniform

  // wave w takes the consecutive units [w*per, (w+1)*per): consecutive
  // chunks of one (sequence, kv-head), a single contiguous stretch of K and
  // V (measured 186 -> 174 us at M = 4 against taking every W-th unit).
  // Paged: the units of the wave's range of pages (paged_worker_range).
  // Wave-uniform by construction; readfirstlane lets the compiler keep the
  // unit (and the descriptors built from it) in scalar registers.
  int u, u_end;
  if constexpr (PAGED) {
    const long long P = paged_pages(a, lane);
    const int F = paged_split_factor(a, P, stride);
    a.chunk *= F;
    if (wid == 0 && lane == 0) *a.x_split = F;   // for the merge
    PagedSpot s0{}, s1{};
    const bool any = paged_worker_range(a, lane, wid, stride, P, s0, s1);
    // every worker with a slot says whether its range starts inside a chunk
    if (wid < a.x_cap && lane == 0) {
      int32_t* mt = a.x_meta + 4 * (size_t)wid;
      mt[0] = s0.b;
      mt[1] = s0.kvh;
      mt[2] = s0.c;
      mt[3] = any && s0.pos % a.chunk != 0 ? 1 : 0;
    }
    if (!any) return;
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
    const int per = (n_units + stride - 1) / stride;
    u = __builtin_amdgcn_readfirstlane(wid * per);
    u_end = min(u + per, n_units);
    if (u >= n_units) return;
  }
  UnitM cur;
  decode(u, cur);
  u32x4 kr[TT][NI], vr[TT][NI];
  int buf = 0;   // LDS copy of the current unit's page ids (paged)
  int pid[kPidPerLane];
  if constexpr (PAGED) {
    page_ids_load(a, cur.b, cur.c0, cur.c1, lane, pid);
    page_ids_store(s_pid[wave][0], lane, pid);
  }
  load_q(cur);
  issue(a.k, cur, buf, cur.c0, cur.c1, kr);
  // The last batch of a unit requests the next unit's query and first K rows
  // before the unit's partials are stored: stores count on the same
  // vector-memory counter as loads, so loads issued after them would wait.
  while (true) {
    const int un = u + 1;
    const bool has_next = un < u_end;
    UnitM nxt = cur;
    if (has_next) decode(un, nxt);
    if constexpr (PAGED) {
      if (has_next) page_ids_load(a, nxt.b, nxt.c0, nxt.c1, lane, pid);
    }
    const int c0 = cur.c0, c1 = cur.c1;
    const int lim = cur.L - a.M + n / G;

    f32x4 o[DB];
    float m = kNegInf, l = 0.f;   // row's running maximum (raw) and this lane's part of l
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int T = c0; T < c1; T += STEP) {
      issue(a.v, cur, buf, T, c1, vr);
      float sc[TT][4];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        // A operand of k-step s: dims 32s + 8 qd .. +8 of row n
        to_lds(lk, kr[tt]);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(lk + n * LSTR + 64 * s + 16 * qd);
          acc = mfma_qk(ka, qf[s], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = T + 16 * tt + 4 * qd + e;
          sc[tt][e] = (pos < c1 && pos <= lim) ? acc[e] : kNegInf;
        }
      }
      // K is requested on every path (after the wave's last batch, this
      // batch's rows again, unused), so the compiler's wait counts agree on
      // all paths and P V waits for this batch's V rows only, not for these
      // loads (measured 189 -> 182 us at M = 4)
      {
        UnitM xs = cur;
        int t_next = T + STEP, c_end = c1, b_next = buf;
        if (T + STEP >= c1 && has_next) {
          load_q(nxt);
          if constexpr (PAGED) page_ids_store(s_pid[wave][buf ^ 1], lane, pid);
          xs = nxt;
          t_next = nxt.c0;
          c_end = nxt.c1;
          b_next = buf ^ 1;
        } else if (T + STEP >= c1) {
          t_next = T;
        }
        issue(a.k, xs, b_next, t_next, c_end, kr);
      }

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
      // P V one tile at a time on v_mfma_f32_16x16x16_bf16 (position 4 qd +
      // e); the pairwise 16x16x32 form measured 3 % slower here (register
      // pressure)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        to_lds(lv, vr[tt]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 vv = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                         (__attribute__((address_space(3))) s16x4_t*)(lv + tr_off + 32 * db)));
          o[db] = mfma_pv(ph[tt], vv, o[db]);
          o[db] = mfma_pv(pl[tt], vv, o[db]);
        }
      }
    }

    // l of row n: the four lanes of the row hold parts
    l = pair_sum<32>(pair_sum<16>(l));
#pragma unroll
    for (int h = 0; h < H; ++h) {
      if (held == h) {   // wave-uniform
        hold_m[h] = m;
        hold_l[h] = l;
#pragma unroll
        for (int db = 0; db < DB; ++db) hold_o[h][db] = o[db];
        hold_x[h] = cur;
      }
    }
    if constexpr (PAGED) {
      // an empty split ran no batch, so nothing requested the next one's
      // query and first K rows yet
      if (c1 <= c0 && has_next) {
        load_q(nxt);
        page_ids_store(s_pid[wave][buf ^ 1], lane, pid);
        issue(a.k, nxt, buf ^ 1, nxt.c0, nxt.c1, kr);
      }
    }
    if (++held == H || !has_next) {
#pragma unroll
      for (int h = 0; h < H; ++h)
        if (h < held) store_unit(hold_o[h], hold_m[h], hold_l[h], hold_x[h]);
      held = 0;
    }
    if (!has_next) break;
    cur = nxt;
    u = un;
    if constexpr (PAGED) buf ^= 1;
  }
}

// Workgroups of this kernel that fit on one compute unit.
template <class K>
static int multi_blocks_per_cu(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0) != hipSuccess ||
      n <= 0)
    n = 1;
  return n;
}

// Units (sequence, kv-head, split) that run at once: one per wave.
template <int D>
size_t multi_wave_slots() {
  static const int per_cu = multi_blocks_per_cu(multi_kernel<D, false>);
  return (size_t)cu_count() * per_cu * kWaves;
}

// *workers: the waves launched (each a worker of a paged call).
template <int D>
hipError_t launch_multi_d(const MultiArgs& a, hipStream_t s, int* workers) {
  // equal rounds for every wave, as for the single-query kernel
  const size_t units = (size_t)a.B * a.Hkv * a.nc;
  const size_t slots = multi_wave_slots<D>();
  const size_t rounds = (units + slots - 1) / slots;
  // paged: every resident wave (the pages are divided over the workers)
  const unsigned grid =
      a.block_table != nullptr
          ? (unsigned)((std::min(units, slots) + kWaves - 1) / kWaves)
          : (unsigned)((units + kWaves * rounds - 1) / (kWaves * rounds));
  *workers = (int)grid * kWaves;
  if (a.block_table != nullptr)
    hipLaunchKernelGGL((multi_kernel<D, true>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((multi_kernel<D, false>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fdk
