// Split-KV decode attention for gfx950: the per-chunk partial kernel (dense,
// paged and fixed-maximum variants) and the exact log-sum-exp merge.
//
// Method: "Flash Decoding" explainer (aiqz.cc), section 2 -- cut the cache
// along the sequence, give every chunk to a different compute unit, keep
// (m_i, l_i, O_i) per chunk, merge with the exp(m_i - m) rescale.  The
// fixed-maximum variant follows the "FlashDecoding" deployment blog,
// section 1 and its fixed_max_value / fallback_on_overflow settings.
//
// Every wavefront owns whole units = (sequence, kv-head, chunk):
//   * A lane holds two 16-byte pieces of a cache row (one for G = 8), so 8
//     lanes share a d = 128 bf16 row and one wave load covers 8 half rows.
//     The K and V loads of a batch overlap the math of the previous one.
//   * QK^T for the G query heads of the kv-head (GQA packing): each lane dots
//     its pieces with the G query pieces (v_dot2c_f32_bf16 for bf16, fp32 FMA
//     for fp32) and a DPP butterfly sums the pieces of a row.
//   * P stays fp32; O accumulates in fp32 (see splitkv.hpp for the row-slot
//     softmax state and the end-of-unit merge).
#include <algorithm>
#include <atomic>

#include "internal.hpp"
#include "splitkv.hpp"

namespace fdk {

constexpr int kMaxChunkPages = 1024;

// 16-byte pieces of a cache row per lane (see Geo in splitkv.hpp).
constexpr int kP = 2;

// Fixed-maximum update with in-flight fallback.  A row slot takes
// p = 2^((s - phi) c) while its running maximum stays inside
// [phi - margin_lo, phi + margin_hi]: no rescale, no dependence on other
// slots or chunks.  The first batch that takes the running maximum out of
// that range switches the slot, for the rest of the chunk, to the exact
// computation with its own maximum: the accumulator is rescaled once from
// phi to that maximum and later batches rescale only when it grows.  Nothing
// is read twice, and a value never meets an exponent outside the range.
// m: running maximum (raw), base: the slot's reference (phi or m, raw),
// on: the slot has switched.
template <typename E, int G, int VEC, int NB, int P>
__device__ __forceinline__ void fixed_update(const float (&s)[NB][G], const u32x4 (&vr)[NB * P],
                                             float c_log2, float phi_raw, float hi_raw,
                                             float lo_raw, float (&acc)[G][VEC], float (&m)[G],
                                             float (&base)[G], bool (&on)[G], float (&l)[G]) {
  float mb[G];
  bool need[G];
  bool change = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mb[h] = m[h];
#pragma unroll
    for (int i = 0; i < NB; ++i) mb[h] = fmaxf(mb[h], s[i][h]);
    const bool out = (mb[h] > hi_raw) || (mb[h] < lo_raw && mb[h] != kNegInf);
    need[h] = on[h] ? (mb[h] > m[h]) : out;
    change |= need[h];
    m[h] = mb[h];
  }
  (void)phi_raw;
  if (__any(change)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (need[h]) {
        const float a = exp2_hw((base[h] - mb[h]) * c_log2);
        l[h] *= a;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] *= a;
        base[h] = mb[h];
        on[h] = true;
      }
    }
  }
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

// One unit of work: chunk c of (sequence b, kv-head kvh), positions [c0, c1).
struct Unit {
  int b, kvh, c, c0, c1;
};

// Split-KV partials.  Work assignment: every wavefront owns whole chunks
// (units) of the flattened (sequence, kv-head, chunk) list: a contiguous
// cache gives wave w the consecutive units [w*per, (w+1)*per), a paged one
// the units w, w + W, w + 2W, ... (W = waves in the grid).  The host sizes
// the grid so that every wave gets the same number of units (the pages'
// advice: a block count that is a multiple of what the cores run at once),
// which keeps each wave's stream of 16-byte loads long and leaves no ragged
// last round.  Row slots of a wave are merged with shuffles; there is no LDS
// combine and no workgroup barrier.
//
// Streaming: a batch is NB rows per row slot.  The V rows of batch j are
// requested before the scores of batch j are computed, and the K rows of the
// next batch before the PV update of batch j -- across unit boundaries too:
// the last batch of a unit requests the next unit's query and first K rows
// (a paged cache has the next unit's page ids staged in LDS by then), and the
// row slots are merged while those loads are in flight.  So a wave's loads
// never stop between its first and its last unit.
template <int MODE, typename E, int D, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void partial_kernel(PartialArgs a) {
  // two pieces per lane halve the per-row work; G = 8 keeps one piece, as
  // its accumulators already fill the registers
  constexpr int kPg = G >= 8 ? 1 : kP;
  using Gm = Geo<E, D, kPg>;
  constexpr int VEC = Gm::kVec, LPT = Gm::kLpt, PV = Gm::kPv, TPL = Gm::kTpl, ROW = Gm::kRow;
  // rows per slot per batch: the batch depth counts load instructions per
  // tensor, and each row takes kPg of them
  constexpr int kNbLoads = batch_rows<G>();
  constexpr int NB = kNbLoads / kPg > 0 ? kNbLoads / kPg : 1;
  constexpr int STEP = NB * TPL;   // rows per wave batch
  constexpr bool kFixed = MODE == kUnified;
  constexpr bool kPagedMode = MODE == kPaged;
  constexpr int kPid = kPagedMode ? kMaxChunkPages : 1;
  // paged: page ids of the current and the next unit of each wave (written
  // and read by that wave only, so no barrier is needed)
  __shared__ int s_pid[kPagedMode ? kWaves : 1][2][kPid];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int col = lane % LPT, grp = lane / LPT;
  const int stride = (int)gridDim.x * kWaves;

  // Units: contiguous caches have B*Hkv*nc equal units.  Paged caches have
  // ragged lengths, so only the real units are numbered: first the whole
  // chunks of every sequence (sequence-major, kv-head fastest; `seq_first` /
  // `seq_units` track the sequence as the wave's unit index grows), then the
  // last, partial chunk of every sequence that has one (one unit per
  // kv-head), longest first when there are at most kMaxSortedSeqs sequences.
  // Waves take units round-robin, so each wave's last round holds the
  // shortest units (longest-processing-time-first order), and the waves
  // finish closer together.  Every numbered unit has c0 < c1.
  constexpr int kMaxSortedSeqs = 128;
  __shared__ int s_tail[kPagedMode ? kWaves : 1][kPagedMode ? kMaxSortedSeqs : 1];
  int n_units = a.B * a.Hkv * a.nc;
  int n_whole = n_units;
  int seq_b = 0, seq_first = 0, seq_units = 0;
  int tail_r = -1, tail_b = -1;
  auto seq_len = [&](int bb) { return min(max(a.seq_lens[bb], 0), a.max_seq_len); };
  // the same for a wave-uniform index, through the scalar cache: its wait
  // is on the LDS/scalar counter, not on the vector-memory counter that the
  // K and V loads in flight hold
  auto seq_len_u = [&](int bb) {
    const auto* sl = (const __attribute__((address_space(4))) int32_t*)a.seq_lens;
    return min(max(sl[__builtin_amdgcn_readfirstlane(bb)], 0), a.max_seq_len);
  };
  const bool sorted_tail = a.B <= kMaxSortedSeqs;
  if constexpr (kPagedMode) {
    int whole = 0, part = 0;
    for (int bb = lane; bb < a.B; bb += kWave) {
      const int L = seq_len(bb);
      whole += L / a.chunk;
      part += L % a.chunk != 0;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      whole += __shfl_xor(whole, o);
      part += __shfl_xor(part, o);
    }
    n_whole = whole * a.Hkv;
    n_units = (whole + part) * a.Hkv;
    seq_units = a.Hkv * (seq_len_u(0) / a.chunk);
    if (sorted_tail) {
      // rank of each partial chunk: longer remainder first, then lower b
      for (int bb = lane; bb < a.B; bb += kWave) {
        const int rem = seq_len(bb) % a.chunk;
        int rank = 0;
        for (int o = 0; o < a.B; ++o) {
          const int ro = seq_len_u(o) % a.chunk;
          rank += ro != 0 && (ro > rem || (ro == rem && o < bb));
        }
        if (rem != 0) s_tail[wave][rank] = bb;
      }
    }
  }
  // sequence of the r-th partial chunk; r grows from call to call
  auto tail_seq = [&](int r) {
    if (sorted_tail) return s_tail[wave][r];
    while (tail_r < r) {      // wave-uniform
      do {
        ++tail_b;
      } while (seq_len_u(tail_b) % a.chunk == 0);
      ++tail_r;
    }
    return tail_b;
  };
  auto decode = [&](int u, Unit& x) {   // u must grow from call to call
    if constexpr (kPagedMode) {
      if (u < n_whole) {
        while (u >= seq_first + seq_units) {      // wave-uniform
          seq_first += seq_units;
          ++seq_b;
          seq_units = a.Hkv * (seq_len_u(seq_b) / a.chunk);
        }
        x.b = seq_b;
        const int r = u - seq_first;
        x.kvh = r % a.Hkv;
        x.c = r / a.Hkv;
        x.c0 = x.c * a.chunk;
        x.c1 = x.c0 + a.chunk;
      } else {
        const int p = u - n_whole;
        x.kvh = p % a.Hkv;
        x.b = tail_seq(p / a.Hkv);
        const int L = seq_len_u(x.b);
        x.c = L / a.chunk;
        x.c0 = x.c * a.chunk;
        x.c1 = L;
      }
    } else {
      x.c = u % a.nc;
      const int bk = u / a.nc;
      x.kvh = bk % a.Hkv;
      x.b = bk / a.Hkv;
      x.c0 = x.c * a.chunk;
      x.c1 = min(x.c0 + a.chunk, a.L);
    }
  };

  // Paged addressing: the page ids of a unit's chunk.
  const int shift = a.page_shift, pmask = (1 << a.page_shift) - 1;
  auto n_pages = [&](const Unit& x) { return (x.c1 - x.c0 + pmask) >> shift; };
  auto page_ids = [&](const Unit& x) {
    return a.block_table + (size_t)x.b * a.max_pages + (x.c0 >> shift);
  };
  auto stage_pages = [&](const Unit& x, int buf) {
    const int npg = n_pages(x);
    const int32_t* bt = page_ids(x);
    for (int i = lane; i < npg; i += kWave) s_pid[wave][buf][i] = min(max(bt[i], 0), a.num_pages - 1);
  };

  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  // Byte offsets (from the tensor base) of this lane's rows of the batch
  // starting at t0; rows past the unit's end repeat its last row (masked).
  auto offsets = [&](const Unit& x, int buf, int t0, size_t (&off)[NB]) {
    const size_t head = kPagedMode ? 0 : ((size_t)x.b * a.Hkv + x.kvh) * (size_t)a.L;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int t = min(t0 + i * TPL + grp, x.c1 - 1);
      size_t row;
      if constexpr (kPagedMode) {
        const int p = min(max(s_pid[wave][buf][(t - x.c0) >> shift], 0), a.num_pages - 1);
        row = (((size_t)p * a.Hkv + x.kvh) << shift) | (size_t)(t & pmask);
      } else {
        row = head + (size_t)t;
      }
      off[i] = row * ROW + (size_t)col * 16;
    }
  };
  // piece pc of row i: bytes off[i] + pc * ROW / kPg; register r[i * kPg + pc]
  auto issue = [&](const char* __restrict__ src, const size_t (&off)[NB],
                   u32x4 (&r)[NB * kPg]) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int pc = 0; pc < kPg; ++pc)
        r[i * kPg + pc] = ld16_stream(src + off[i] + (size_t)pc * (ROW / kPg));
  };
  // Contiguous caches: a batch of the tensor at `src`
  // starting at row t0 of unit x is read through one buffer descriptor whose
  // base is that row and whose byte limit ends at the unit's end c1, so rows
  // past c1 read as zeros without touching memory (their scores are masked,
  // their p is 0).  Load (i, pc) of this lane sits at byte
  // i * TPL * ROW + pc * ROW / kPg + grp * ROW + col * 16 of the batch: the
  // multiple of 4096 comes from one of kNvo lane offsets fixed for the whole
  // kernel, the rest is the instruction's immediate, so the batch costs no
  // per-load address arithmetic.  The range check covers the lane offset
  // plus the immediate.
  constexpr int kBatchBytes = STEP * ROW;
  constexpr int kNvo = (kBatchBytes + 4095) / 4096;
  int lane_voff[kNvo];
#pragma unroll
  for (int j = 0; j < kNvo; ++j) lane_voff[j] = j * 4096 + grp * ROW + col * 16;
  auto issue_c = [&](const char* __restrict__ src, const Unit& x, int t0,
                     u32x4 (&r)[NB * kPg]) {
    const size_t head = ((size_t)x.b * a.Hkv + x.kvh) * (size_t)a.L;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(src + (head + (size_t)t0) * ROW, min(x.c1 - t0, STEP) * ROW);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int pc = 0; pc < kPg; ++pc) {
        constexpr int kPcBytes = ROW / kPg;
        const int byte = i * TPL * ROW;
        r[i * kPg + pc] = ld16_buf(rs, lane_voff[byte / 4096] + byte % 4096 + pc * kPcBytes);
      }
  };
  constexpr bool kBufC = !kPagedMode;
  u32x4 qv[G][kPg];
  auto load_q = [&](const Unit& x) {
    const E* qp = reinterpret_cast<const E*>(a.q) +
                  ((size_t)x.b * a.Hq + (size_t)x.kvh * G) * D + col * PV;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int pc = 0; pc < kPg; ++pc) qv[h][pc] = ld16(qp + (size_t)h * D + pc * (D / kPg));
  };
  auto scores = [&](const Unit& x, int t0, const u32x4 (&kr)[NB * kPg], float (&s)[NB][G]) {
    float flat[NB * G];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) flat[i * G + h] = pieces_dot<E, kPg>(qv[h], kr + i * kPg);
    group_sum_n<LPT>(flat);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) s[i][h] = flat[i * G + h];
    if (t0 + STEP > x.c1) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (t0 + i * TPL + grp >= x.c1)
#pragma unroll
          for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
    }
  };

  // Finished units wait (in LDS) until H are held or the wave runs out of
  // units, and are then written together.  Stores count on the same
  // vector-memory counter as loads, so a store issued between units would
  // make the next unit's first loads wait for it (measured: 11 us of 169 on
  // the 1 GiB workload).  After the reduce-scatter every lane has NK values
  // of the unit and NCOPY lanes have the same ones, so the copies take turns:
  // held unit j stays in slot j / NCOPY of s_keep for the lanes with copy
  // index j % NCOPY, which also write it.  The unit's (m, l) and flags stay
  // with the lanes of row slot j.
  using SS = SlotScatter<LPT, G, VEC>;
  constexpr int NK = SS::NK, NCOPY = SS::NCOPY;
  constexpr int NSLOT = 64 / NK;   // units held per lane (64 values)
  constexpr int H = TPL < NSLOT * NCOPY ? TPL : NSLOT * NCOPY;
  const int cpy = SS::copy(lane);
  constexpr int NSLOTS = (H + NCOPY - 1) / NCOPY;
  // held values in LDS (lane-major 16-byte groups: conflict-free), which
  // keeps the batch loop's working set in the vector registers (headline step
  // 167.8 -> 166.4 us against holding them in registers)
  __shared__ __align__(16) f32x4 s_keep[kWaves][NSLOTS][NK / 4][kWave];
  float keep_m[G], keep_l[G];
  size_t keep_rows[H];
  size_t keep_row_ml = 0;
  unsigned keep_flags = 0;
  int held = 0;   // wave-uniform
  auto flush = [&]() {
#pragma unroll
    for (int j = 0; j < H; ++j) {
      if (j < held && cpy == j % NCOPY) {
#pragma unroll
        for (int k = 0; k < NK; k += 4) {
          const int K = SS::index(lane, k);
          const int h = K / VEC, e = K % VEC;
          float* dst = a.o_part + (keep_rows[j] + (size_t)h * a.nc) * D + Gm::dim(col, e);
          *reinterpret_cast<f32x4*>(dst) = s_keep[wave][j / NCOPY][k / 4][lane];
        }
      }
    }
    if (grp < held) {
      if (col == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
          *reinterpret_cast<f32x2*>(a.ml_part + (keep_row_ml + (size_t)h * a.nc) * 2) =
              f32x2{keep_m[h], keep_l[h]};
      }
      if constexpr (kFixed) {
        if (a.flags != nullptr && col < G)
          a.flags[keep_row_ml + (size_t)col * a.nc] = (uint8_t)((keep_flags >> col) & 1u);
      }
    }
    held = 0;
  };

  // Contiguous caches: wave w takes the consecutive units [w*per, (w+1)*per)
  // -- consecutive chunks of one (sequence, kv-head), a single contiguous
  // stretch of K and V (measured 162.7 -> 161.6 us against taking every
  // W-th unit).  Paged caches keep the round-robin order above, whose last
  // round holds the shortest units.
  const int per = kPagedMode ? 1 : (n_units + stride - 1) / stride;
  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // unit (and the buffer descriptors built from it) in scalar registers
  int u = __builtin_amdgcn_readfirstlane(((int)blockIdx.x * kWaves + wave) * per);
  const int u_end = kPagedMode ? n_units : min(u + per, n_units);
  const int ustep = kPagedMode ? stride : 1;
  if (u >= n_units) return;
  Unit cur;
  decode(u, cur);
  int buf = 0;
  if constexpr (kPagedMode) stage_pages(cur, buf);
  u32x4 kr[NB * kPg], vr[NB * kPg];
  size_t off[NB];
  load_q(cur);
  if constexpr (kBufC) {
    issue_c(kbase, cur, cur.c0, kr);
  } else {
    offsets(cur, buf, cur.c0, off);
    issue(kbase, off, kr);
  }

  while (true) {
    const int un = u + ustep;
    const bool has_next = un < u_end;   // wave-uniform
    Unit nxt = cur;
    if (has_next) decode(un, nxt);
    // paged: the next unit's page ids, one per lane when they fit (written
    // to LDS once the first batch of this unit has arrived)
    int pid_next = 0;
    bool pid_inline = false;
    if constexpr (kPagedMode) {
      if (has_next) {
        const int npg = n_pages(nxt);
        pid_inline = npg <= kWave;
        if (pid_inline && lane < npg) pid_next = page_ids(nxt)[lane];
      }
    }

    float acc[G][VEC], m[G], l[G], mx[G], base[G];
    bool on[G];
    state_reset<G, VEC>(acc, m, l);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = kNegInf;
      base[h] = a.phi_raw;
      on[h] = false;
    }
    // every unit has at least one row (c0 < c1): a loop without a zero-trip
    // path, so that no load issued above looks pending at the unit's end
    int t0 = cur.c0;
    do {
      if constexpr (kBufC) issue_c(vbase, cur, t0, vr);
      else issue(vbase, off, vr);
      float s[NB][G];
      scores(cur, t0, kr, s);
      if constexpr (kPagedMode) {
        if (has_next && t0 == cur.c0) {
          if (pid_inline) {
            if (lane < n_pages(nxt)) s_pid[wave][buf ^ 1][lane] = pid_next;
          } else {
            stage_pages(nxt, buf ^ 1);
          }
        }
      }
      if (t0 + STEP < cur.c1) {
        if constexpr (kBufC) {
          issue_c(kbase, cur, t0 + STEP, kr);
        } else {
          offsets(cur, buf, t0 + STEP, off);
          issue(kbase, off, kr);
        }
      } else if (has_next) {
        load_q(nxt);
        if constexpr (kBufC) {
          issue_c(kbase, nxt, nxt.c0, kr);
        } else {
          offsets(nxt, buf ^ 1, nxt.c0, off);
          issue(kbase, off, kr);
        }
      }
      if constexpr (kFixed)
        fixed_update<E, G, VEC, NB, kPg>(s, vr, a.c_log2, a.phi_raw, a.flag_hi_raw,
                                         a.flag_lo_raw, acc, mx, base, on, l);
      else online_update<E, G, VEC, NB, kPg>(s, vr, a.c_log2, acc, m, l);
      t0 += STEP;
    } while (t0 < cur.c1);
    // m in log2 units of the scaled score: the slot's own maximum, or for
    // the fixed maximum its reference (phi, or its own maximum after a
    // switch); a slot that saw no row has m = -inf, l = 0
    unsigned flag_bits = 0;
    if constexpr (kFixed) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m[h] = (mx[h] == kNegInf) ? kNegInf : base[h] * a.c_log2;
        // range flag of each head's chunk maximum (slots that left the range
        // already finished the chunk on the exact path)
        const float mm = wave_max(mx[h]);
        if ((mm > a.flag_hi_raw) || (mm < a.flag_lo_raw)) flag_bits |= 1u << h;
      }
    } else {
      state_to_log2<G>(m, a.c_log2);
    }

    float kept[NK];
    slot_reduce_scatter<LPT, G, VEC>(acc, m, l, kept);
    const size_t row0 = ((size_t)cur.b * a.Hq + (size_t)cur.kvh * G) * a.nc + cur.c;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      if (held == j) {   // wave-uniform
        if (cpy == j % NCOPY) {
#pragma unroll
          for (int k = 0; k < NK; k += 4)
            s_keep[wave][j / NCOPY][k / 4][lane] =
                f32x4{kept[k], kept[k + 1], kept[k + 2], kept[k + 3]};
        }
        keep_rows[j] = row0;
      }
    }
    if (grp == held) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        keep_m[h] = m[h];
        keep_l[h] = l[h];
      }
      keep_row_ml = row0;
      keep_flags = flag_bits;
    }
    if (++held == H) flush();
    if (!has_next) break;
    cur = nxt;
    u = un;
    buf ^= 1;
  }
  flush();
}

// Exact merge of a row's chunk partials ("Flash Decoding" explainer,
// section 2, steps 2-4, with unnormalised O_i):
//   M = max_i m_i,  w_i = 2^(m_i - M),
//   out = sum_i w_i O_i / sum_i w_i l_i,  lse = (M + log2 sum_i w_i l_i) ln 2.
// A row whose chunks are all empty (a query token of a paged sequence
// shorter than its position) has sum_i w_i l_i = 0: out = 0, lse = -inf,
// the empty softmax.
// This kernel takes rows of more than 256 chunks (shorter rows take
// merge_wave_kernel below): one workgroup of W waves per (sequence, query
// head, slice of D / CS columns), so that more loads share one memory
// latency.  The weights of up to 64 W chunks at a time go to LDS; thread
// (chunk lane cl, column group cg) then sums chunks cl, cl + CL, ... of 4
// columns with independent 16-byte loads, 16 W CS chunks at a time (the
// loads of the first group are issued before the maximum is known), and the
// chunk lanes are reduced through LDS.  The order of every sum is fixed, so
// runs are bitwise reproducible.  Rows whose chunks all carry the same m (the fixed-maximum
// path without fallback) get weights of exactly 1.
template <int D, int W, int CS>
__global__ __launch_bounds__(W * kWave) void merge_kernel(MergeArgs a) {
  constexpr int kMergeThreads = W * kWave;
  constexpr int CG = D / 4 / CS;        // 16-byte column groups of this workgroup's columns
  constexpr int CL = kMergeThreads / CG;     // chunk lanes
  constexpr int kPre = 16 * W * CS / CL > 0 ? 16 * W * CS / CL : 1;   // chunks up front, per lane
  __shared__ float s_red[W];
  __shared__ float s_w[kMergeThreads];
  __shared__ f32x4 s_o[CL][CG];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & (kWave - 1);
  const int cl = tid / CG, cg = tid % CG;
  const size_t row = blockIdx.x / CS;
  const int cs = (int)(blockIdx.x % CS);   // this workgroup's share of the columns
  int n = a.nc;
  if (a.seq_lens != nullptr) {
    const int b = (int)(row / a.Hq);
    const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
    const int split = a.chunk_scale != nullptr ? a.chunk * min(max(*a.chunk_scale, 1), 256)
                                               : a.chunk;
    n = min((int)(((long long)L + split - 1) / split), a.nc);
  }
  if (n == 0) {
    if (tid < D / CS) a.out[row * D + cs * (D / CS) + tid] = 0.f;
    if (tid == 0 && cs == 0 && a.lse != nullptr) a.lse[row] = kNegInf;
    return;
  }
  // column group cg of this workgroup is column group cs * CG + cg of the row;
  // chunk k's groups start at op[k * (D / 4)]
  const f32x4* op = reinterpret_cast<const f32x4*>(a.o_part + row * a.nc * D) + cs * CG;
  const f32x2* mlp = reinterpret_cast<const f32x2*>(a.ml_part + row * a.nc * 2);

  // Everything the first kPre * CL chunks need is requested before any
  // arithmetic, so the (m, l) and O loads share one memory latency.
  f32x4 pre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int k = cl + j * CL;
    pre[j] = k < n ? op[(size_t)k * (D / 4) + cg] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const f32x2 ml0 = tid < n ? mlp[tid] : f32x2{kNegInf, 0.f};

  float mx = ml0.x;
  for (int c = tid + kMergeThreads; c < n; c += kMergeThreads) mx = fmaxf(mx, mlp[c].x);
  mx = wave_max(mx);
  if (lane == 0) s_red[w] = mx;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int i = 1; i < W; ++i) M = fmaxf(M, s_red[i]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float ls = 0.f;
  for (int c0 = 0; c0 < n; c0 += kMergeThreads) {
    const int c = c0 + tid;
    float wt = 0.f;
    if (c < n) {
      const f32x2 mlc = c0 == 0 ? ml0 : mlp[c];
      wt = exp2_diff(mlc.x, M);
      ls = fmaf(wt, mlc.y, ls);
    }
    __syncthreads();   // previous tile's s_w reads are done
    s_w[tid] = wt;
    __syncthreads();
    const int nt = min(kMergeThreads, n - c0);
    // groups of kPre chunks per thread: all loads of a group are issued
    // before its sums (the first group of the first tile is already loaded)
    for (int k0 = 0; k0 < nt; k0 += kPre * CL) {
      f32x4 o[kPre];
      if (c0 == 0 && k0 == 0) {
#pragma unroll
        for (int j = 0; j < kPre; ++j) o[j] = pre[j];
      } else {
#pragma unroll
        for (int j = 0; j < kPre; ++j) {
          const int k = k0 + cl + j * CL;
          o[j] = k < nt ? op[(size_t)(c0 + k) * (D / 4) + cg] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int j = 0; j < kPre; ++j) {
        const int k = k0 + cl + j * CL;
        if (k < nt) {
          const float x = s_w[k];
          acc.x = fmaf(x, o[j].x, acc.x);
          acc.y = fmaf(x, o[j].y, acc.y);
          acc.z = fmaf(x, o[j].z, acc.z);
          acc.w = fmaf(x, o[j].w, acc.w);
        }
      }
    }
  }
  s_o[cl][cg] = acc;
  ls = wave_sum(ls);
  __syncthreads();
  if (lane == 0) s_red[w] = ls;
  __syncthreads();
  if (tid < CG) {
    f32x4 t = s_o[0][tid];
#pragma unroll
    for (int k = 1; k < CL; ++k) {
      const f32x4 u = s_o[k][tid];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < W; i += 2) den += s_red[i] + s_red[i + 1];
    reinterpret_cast<f32x4*>(a.out + row * D)[cs * CG + tid] =
        den > 0.f ? f32x4{t.x / den, t.y / den, t.z / den, t.w / den} : f32x4{0.f, 0.f, 0.f, 0.f};
    if (tid == 0 && cs == 0 && a.lse != nullptr) a.lse[row] = (M + log2_hw(den)) * kLn2;
  }
}

// The same merge for rows of at most 64 NM chunks on one wavefront per
// (row, column slice of D / CS floats), with no barrier and no LDS: lane c
// holds the (m, l) of chunks c, c + 64, ... (NM of them), the maximum and
// the denominator are wave reductions, lane (cl, cg) sums chunks cl,
// cl + CL, ... of its 4 columns (every O load issued before the maximum is
// known) with the weights taken from the chunks' lanes, and the CL chunk
// lanes of a column group add up through pair exchanges.  Fixed summation
// order.
template <int D, int CS, int NM>
__global__ __launch_bounds__(kWave) void merge_wave_kernel(MergeArgs a) {
  constexpr int CG = D / 4 / CS;        // 16-byte column groups of the slice
  constexpr int CL = kWave / CG;        // chunk lanes
  constexpr int KP = kWave * NM / CL;   // chunks per lane
  static_assert(CL == 2 || CL == 4 || CL == 8 || CL == 16, "chunk lanes");
  const int lane = threadIdx.x;
  const int cl = lane / CG, cg = lane % CG;
  const size_t row = blockIdx.x / CS;
  const int cs = (int)(blockIdx.x % CS);
  int n = a.nc;
  if (a.seq_lens != nullptr) {
    const int b = (int)(row / a.Hq);
    const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
    const int split = a.chunk_scale != nullptr ? a.chunk * min(max(*a.chunk_scale, 1), 256)
                                               : a.chunk;
    n = min((int)(((long long)L + split - 1) / split), a.nc);
  }
  if (n == 0) {   // wave-uniform
    for (int c = lane; c < D / CS; c += kWave) a.out[row * D + cs * (D / CS) + c] = 0.f;
    if (lane == 0 && cs == 0 && a.lse != nullptr) a.lse[row] = kNegInf;
    return;
  }
  const f32x4* op = reinterpret_cast<const f32x4*>(a.o_part + row * a.nc * D) + cs * CG + cg;
  const f32x2* mlp = reinterpret_cast<const f32x2*>(a.ml_part + row * a.nc * 2);
  f32x4 o[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const int k = cl + j * CL;
    o[j] = k < n ? op[(size_t)k * (D / 4)] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f32x2 ml[NM];
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    const int k = lane + i * kWave;
    ml[i] = k < n ? mlp[k] : f32x2{kNegInf, 0.f};
    mx = fmaxf(mx, ml[i].x);
  }
  const float M = wave_max(mx);
  float w[NM], ls = 0.f;
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    w[i] = lane + i * kWave < n ? exp2_diff(ml[i].x, M) : 0.f;
    ls = fmaf(w[i], ml[i].y, ls);
  }
  const float den = wave_sum(ls);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    // chunk k = cl + j CL sits in lane k % 64 of weight set k / 64, the same
    // set in every lane (CL divides 64)
    const int k = cl + j * CL;
    const float wk = __shfl(w[j * CL / kWave], k % kWave);
    acc.x = fmaf(wk, o[j].x, acc.x);
    acc.y = fmaf(wk, o[j].y, acc.y);
    acc.z = fmaf(wk, o[j].z, acc.z);
    acc.w = fmaf(wk, o[j].w, acc.w);
  }
  // chunk lane cl of column group cg is lane cl * CG + cg
  auto sum_lanes = [&](float x) {
    if constexpr (CL >= 16) x = pair_sum<4>(x);
    if constexpr (CL >= 8) x = pair_sum<8>(x);
    if constexpr (CL >= 4) x = pair_sum<16>(x);
    return pair_sum<32>(x);
  };
  acc.x = sum_lanes(acc.x);
  acc.y = sum_lanes(acc.y);
  acc.z = sum_lanes(acc.z);
  acc.w = sum_lanes(acc.w);
  if (cl == 0)
    reinterpret_cast<f32x4*>(a.out + row * D)[cs * CG + cg] =
        den > 0.f ? f32x4{acc.x / den, acc.y / den, acc.z / den, acc.w / den}
                  : f32x4{0.f, 0.f, 0.f, 0.f};
  if (lane == 0 && cs == 0 && a.lse != nullptr) a.lse[row] = (M + log2_hw(den)) * kLn2;
}

int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups of this kernel that fit on one compute unit.
template <class K>
static int blocks_per_cu(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0) != hipSuccess ||
      n <= 0)
    n = 1;
  return n;
}

// Grid for `units` wave-sized units: the fewest equal rounds the resident
// waves allow, and just enough workgroups for them.
static unsigned unit_grid(int per_cu, size_t units) {
  const size_t slots = (size_t)cu_count() * per_cu * kWaves;
  const size_t rounds = (units + slots - 1) / slots;
  return (unsigned)((units + kWaves * rounds - 1) / (kWaves * rounds));
}

template <int MODE, typename E, int D, int G>
static hipError_t launch_p4(const PartialArgs& a, hipStream_t s) {
  auto kernel = partial_kernel<MODE, E, D, G>;
  static const int per_cu = blocks_per_cu(kernel);   // one per instantiation
  const size_t units = (size_t)a.B * a.Hkv * a.nc;
  // Paged: the number of real units is known only on the device, so every
  // resident wave takes part (at most `units` waves).
  const unsigned grid = MODE == kPaged
      ? (unsigned)std::min<size_t>((size_t)cu_count() * per_cu, (units + kWaves - 1) / kWaves)
      : unit_grid(per_cu, units);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int MODE, typename E, int D>
static hipError_t launch_p3(int G, const PartialArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return launch_p4<MODE, E, D, 1>(a, s);
    case 2: return launch_p4<MODE, E, D, 2>(a, s);
    case 4: return launch_p4<MODE, E, D, 4>(a, s);
    case 8: return launch_p4<MODE, E, D, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int MODE>
static hipError_t launch_p2(int is_bf16, int D, int G, const PartialArgs& a, hipStream_t s) {
  if (is_bf16) {
    if (D == 64) return launch_p3<MODE, uint16_t, 64>(G, a, s);
    if (D == 128) return launch_p3<MODE, uint16_t, 128>(G, a, s);
  } else {
    if (D == 64) return launch_p3<MODE, float, 64>(G, a, s);
    if (D == 128) return launch_p3<MODE, float, 128>(G, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_partial(int mode, int is_bf16, int D, int G, const PartialArgs& a,
                          hipStream_t s) {
  switch (mode) {
    case kDense: return launch_p2<kDense>(is_bf16, D, G, a, s);
    case kPaged: return launch_p2<kPaged>(is_bf16, D, G, a, s);
    case kUnified: return launch_p2<kUnified>(is_bf16, D, G, a, s);
  }
  return hipErrorInvalidValue;
}

// Range flags of the fixed maximum from chunk partials (the chunks' own
// maxima): one thread per (sequence, head, chunk).
__global__ __launch_bounds__(256) void range_flags_kernel(const float* ml, uint8_t* flags,
                                                         size_t n, float hi, float lo) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float m = ml[2 * i];
  flags[i] = (uint8_t)((m > hi || m < lo) ? 1 : 0);
}

hipError_t launch_range_flags(const float* ml, uint8_t* flags, size_t n, float hi, float lo,
                              hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(range_flags_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ml,
                     flags, n, hi, lo);
  return hipGetLastError();
}

hipError_t launch_merge(int D, int B, const MergeArgs& a, hipStream_t s) {
  const size_t rows = (size_t)B * a.Hq;
  // rows of at most 256 chunks: one wave per (row, column slice), 16 chunks
  // per lane (32 for d = 128 up to 32 chunks)
  if (a.nc <= 256 && (D == 64 || D == 128)) {
    const dim3 blk(kWave);
    if (D == 128) {
      if (a.nc <= 32)
        hipLaunchKernelGGL((merge_wave_kernel<128, 1, 1>), dim3((unsigned)rows), blk, 0, s, a);
      else if (a.nc <= 64)
        hipLaunchKernelGGL((merge_wave_kernel<128, 2, 1>), dim3((unsigned)(rows * 2)), blk, 0, s, a);
      else if (a.nc <= 128)
        hipLaunchKernelGGL((merge_wave_kernel<128, 4, 2>), dim3((unsigned)(rows * 4)), blk, 0, s, a);
      else
        hipLaunchKernelGGL((merge_wave_kernel<128, 8, 4>), dim3((unsigned)(rows * 8)), blk, 0, s, a);
    } else {
      if (a.nc <= 64)
        hipLaunchKernelGGL((merge_wave_kernel<64, 1, 1>), dim3((unsigned)rows), blk, 0, s, a);
      else if (a.nc <= 128)
        hipLaunchKernelGGL((merge_wave_kernel<64, 2, 2>), dim3((unsigned)(rows * 2)), blk, 0, s, a);
      else
        hipLaunchKernelGGL((merge_wave_kernel<64, 4, 4>), dim3((unsigned)(rows * 4)), blk, 0, s, a);
    }
    return hipGetLastError();
  }
  // Longer rows: one workgroup of 4 waves per (row, quarter of the
  // columns), walking the chunks in tiles of 256.
  const dim3 grid((unsigned)(rows * 4)), block(4 * kWave);
  if (D == 64) hipLaunchKernelGGL((merge_kernel<64, 4, 4>), grid, block, 0, s, a);
  else if (D == 128) hipLaunchKernelGGL((merge_kernel<128, 4, 4>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fdk
