// Split-KV decode attention for gfx950: the per-chunk partial kernel (dense,
// paged and fixed-maximum variants) and the exact log-sum-exp merge.
//
// Method: "Flash Decoding" explainer (aiqz.cc), section 2 -- cut the cache
// along the sequence, give every chunk to a different compute unit, keep
// (m_i, l_i, O_i) per chunk, merge with the exp(m_i - m) rescale.  The
// fixed-maximum variant follows the "FlashDecoding" deployment blog,
// section 1 and its fixed_max_value / fallback_on_overflow settings.
//
// One workgroup = one unit = (sequence, kv-head, chunk):
//   * 4 wavefronts split the chunk into 4 contiguous ranges of rows.
//   * Each lane reads 16 bytes per row; one wave load covers kTpl rows
//     (4 rows of a d = 128 bf16 cache, 1 KiB of contiguous HBM).  The K and V
//     rows of a batch of kNb loads are issued together before any math.
//   * QK^T for the G query heads of the kv-head (GQA packing): each lane dots
//     its slice with the G query slices (v_dot2c_f32_bf16 for bf16, fp32 FMA
//     for fp32) and a DPP butterfly sums the slices of a row.
//   * P stays fp32; O accumulates in fp32 (see splitkv.hpp for the row-slot
//     softmax state and the end-of-unit combine).
#include "internal.hpp"
#include "splitkv.hpp"

namespace fdk {

constexpr int kMaxChunkPages = 1024;

// Byte offset (in rows) of cache position t for one kv-head.
struct RowMap {
  const int* pid;   // paged: LDS page ids of the chunk, else null
  int c0;           // first position of the chunk
  int shift;        // log2(page size)
  int hkv, kvh;
  __device__ __forceinline__ size_t row(int t) const {
    if (pid == nullptr) return (size_t)t;
    const int p = pid[(t - c0) >> shift];
    return ((size_t)(p * hkv + kvh) << shift) | (size_t)(t & ((1 << shift) - 1));
  }
};

// Fixed-maximum update: p = 2^(s*c - base), no running maximum and no
// rescale; the largest raw score is tracked only for the range check.
template <typename E, int G, int VEC>
__device__ __forceinline__ void fixed_update(const float (&s)[kNb][G], const u32x4 (&vr)[kNb],
                                             float c_log2, float base_log2,
                                             float (&acc)[G][VEC], float (&mx)[G],
                                             float (&l)[G]) {
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < kNb; ++i) mx[h] = fmaxf(mx[h], s[i][h]);
#pragma unroll
  for (int i = 0; i < kNb; ++i) {
    float vf[VEC];
    slice_vals<E>(vr[i], vf);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = exp2_hw(fmaf(s[i][h], c_log2, -base_log2));
      l[h] += p;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
    }
  }
}

// Stream rows [t_beg, t_end) of one kv-head through the G query heads.  On
// return m[h] is in log2 units of the scaled score: the slot's own maximum
// (FIXED = false) or base_log2 (FIXED = true, where mx[h] receives the largest
// raw dot product for the range check).
template <bool FIXED, typename E, int D, int G>
__device__ __forceinline__ void scan_rows(const char* __restrict__ kb,
                                          const char* __restrict__ vb, const RowMap& rm,
                                          int t_beg, int t_end, const u32x4 (&qv)[G],
                                          float c_log2, float base_log2,
                                          float (&acc)[G][Geo<E, D>::kVec], float (&m)[G],
                                          float (&l)[G], float (&mx)[G]) {
  using Gm = Geo<E, D>;
  constexpr int LPT = Gm::kLpt, TPL = Gm::kTpl, ROW = Gm::kRow;
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane / LPT, col = lane % LPT;
  state_reset<G, Gm::kVec>(acc, m, l);
#pragma unroll
  for (int h = 0; h < G; ++h) mx[h] = kNegInf;

  for (int t0 = t_beg; t0 < t_end; t0 += kNb * TPL) {
    size_t off[kNb];
#pragma unroll
    for (int i = 0; i < kNb; ++i) {
      const int t = min(t0 + i * TPL + grp, t_end - 1);
      off[i] = rm.row(t) * ROW + (size_t)col * 16;
    }
    u32x4 kr[kNb], vr[kNb];
#pragma unroll
    for (int i = 0; i < kNb; ++i) kr[i] = ld16(kb + off[i]);
#pragma unroll
    for (int i = 0; i < kNb; ++i) vr[i] = ld16(vb + off[i]);

    float s[kNb][G];
#pragma unroll
    for (int i = 0; i < kNb; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) s[i][h] = group_sum<LPT>(slice_dot<E>(qv[h], kr[i]));
    if (t0 + kNb * TPL > t_end) {
#pragma unroll
      for (int i = 0; i < kNb; ++i)
        if (t0 + i * TPL + grp >= t_end)
#pragma unroll
          for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
    }
    if constexpr (FIXED) fixed_update<E, G, Gm::kVec>(s, vr, c_log2, base_log2, acc, mx, l);
    else online_update<E, G, Gm::kVec>(s, vr, c_log2, acc, m, l);
  }
  if constexpr (FIXED) {
#pragma unroll
    for (int h = 0; h < G; ++h) m[h] = base_log2;
  } else {
    state_to_log2<G>(m, c_log2);
  }
}

template <int MODE, typename E, int D, int G>
__global__ __launch_bounds__(kThreads) void partial_kernel(PartialArgs a) {
  using Gm = Geo<E, D>;
  constexpr int VEC = Gm::kVec, LPT = Gm::kLpt, TPL = Gm::kTpl;
  constexpr bool kFixed = MODE == kUnified;
  __shared__ CombineLds<G, D> s_cmb;
  __shared__ float s_mx[kWaves][G];
  __shared__ int s_pid[MODE == kPaged ? kMaxChunkPages : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
  const int col = lane % LPT;
  const int c = blockIdx.x % a.nc;
  const int bk = blockIdx.x / a.nc;
  const int kvh = bk % a.Hkv, b = bk / a.Hkv;

  int L = a.L;
  if constexpr (MODE == kPaged) L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int c0 = c * a.chunk;
  if (c0 >= L) return;  // whole workgroup: chunk past this sequence's end
  const int c1 = min(c0 + a.chunk, L);

  RowMap rm{nullptr, c0, a.page_shift, a.Hkv, kvh};
  const char* kb;
  const char* vb;
  if constexpr (MODE == kPaged) {
    const int first = c0 >> a.page_shift;
    const int npg = (c1 - c0 + (1 << a.page_shift) - 1) >> a.page_shift;
    const int32_t* bt = a.block_table + (size_t)b * a.max_pages + first;
    for (int i = tid; i < npg; i += kThreads) s_pid[i] = min(max(bt[i], 0), a.num_pages - 1);
    __syncthreads();
    rm.pid = s_pid;
    kb = reinterpret_cast<const char*>(a.k);
    vb = reinterpret_cast<const char*>(a.v);
  } else {
    const size_t base = ((size_t)b * a.Hkv + kvh) * (size_t)a.L * Gm::kRow;
    kb = reinterpret_cast<const char*>(a.k) + base;
    vb = reinterpret_cast<const char*>(a.v) + base;
  }

  // This wave's rows: a quarter of the chunk, rounded up to whole loads.
  const int n = c1 - c0;
  const int per = (((n + kWaves - 1) / kWaves) + TPL - 1) / TPL * TPL;
  const int t_beg = c0 + wave * per;
  const int t_end = min(t_beg + per, c1);

  u32x4 qv[G];
  {
    const E* qp = reinterpret_cast<const E*>(a.q) +
                  ((size_t)b * a.Hq + (size_t)kvh * G) * D + col * VEC;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = ld16(qp + (size_t)h * D);
  }

  float acc[G][VEC], m[G], l[G], mx[G];
  scan_rows<kFixed, E, D, G>(kb, vb, rm, t_beg, t_end, qv, a.c_log2, a.base_log2, acc, m, l,
                             mx);

  if constexpr (kFixed) {
    // Range check of each head's chunk maximum.  Any head out of range sends
    // the whole unit through the exact path (its own maximum), which is the
    // fallback recompute; its flag is reported.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w = wave_max(mx[h]);
      if (lane == 0) s_mx[wave][h] = w;
    }
    __syncthreads();
    bool any = false;
    bool flag[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mm = fmaxf(fmaxf(s_mx[0][h], s_mx[1][h]), fmaxf(s_mx[2][h], s_mx[3][h]));
      flag[h] = (mm > a.flag_hi_raw) || (mm < a.flag_lo_raw);
      any |= flag[h];
    }
    if (a.flags != nullptr && tid < G) {
      bool f = false;
#pragma unroll
      for (int h = 0; h < G; ++h) f = (h == tid) ? flag[h] : f;
      a.flags[((size_t)b * a.Hq + (size_t)kvh * G + tid) * a.nc + c] = f ? 1 : 0;
    }
    if (any)
      scan_rows<false, E, D, G>(kb, vb, rm, t_beg, t_end, qv, a.c_log2, a.base_log2, acc, m,
                                l, mx);
  }

  const size_t prow0 = ((size_t)b * a.Hq + (size_t)kvh * G) * a.nc + c;
  combine_store<G, D, VEC, LPT>(s_cmb, acc, m, l, a.o_part, a.ml_part, prow0, (size_t)a.nc);
}

// Exact merge of a row's chunk partials ("Flash Decoding" explainer,
// section 2, steps 2-4, with unnormalised O_i):
//   M = max_i m_i,  w_i = 2^(m_i - M),
//   out = sum_i w_i O_i / sum_i w_i l_i,  lse = (M + log2 sum_i w_i l_i) ln 2.
// One workgroup per (sequence, query head); wave w takes chunks w, w+4, ...
// and every lane D/64 dims.  The summation order is fixed, so runs are
// bitwise reproducible.  Rows whose chunks all carry the same m (the
// fixed-maximum path without fallback) get weights of exactly 1: a plain sum.
template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  constexpr int VPT = D / kWave;
  __shared__ float s_m[kWaves];
  __shared__ float s_l[kWaves];
  __shared__ float s_o[kWaves][D];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & (kWave - 1);
  const size_t row = blockIdx.x;
  int n = a.nc;
  if (a.seq_lens != nullptr) {
    const int b = (int)(row / a.Hq);
    const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
    n = min((L + a.chunk - 1) / a.chunk, a.nc);
  }
  if (n == 0) {
    if (tid < D) a.out[row * D + tid] = 0.f;
    if (tid == 0 && a.lse != nullptr) a.lse[row] = kNegInf;
    return;
  }
  const float* ml = a.ml_part + row * a.nc * 2;
  const float* op = a.o_part + row * a.nc * D;

  float mx = kNegInf;
  for (int c = tid; c < n; c += kThreads) mx = fmaxf(mx, ml[2 * c]);
  mx = wave_max(mx);
  if (lane == 0) s_m[w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));

  float o[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) o[v] = 0.f;
  float ls = 0.f;
  for (int c = w; c < n; c += kWaves) {
    const float wt = exp2_diff(ml[2 * c], M);
    ls = fmaf(wt, ml[2 * c + 1], ls);
#pragma unroll
    for (int v = 0; v < VPT; ++v) o[v] = fmaf(wt, op[(size_t)c * D + lane * VPT + v], o[v]);
  }
#pragma unroll
  for (int v = 0; v < VPT; ++v) s_o[w][lane * VPT + v] = o[v];
  if (lane == 0) s_l[w] = ls;
  __syncthreads();
  if (tid < D) {
    const float den = (s_l[0] + s_l[1]) + (s_l[2] + s_l[3]);
    const float num = (s_o[0][tid] + s_o[1][tid]) + (s_o[2][tid] + s_o[3][tid]);
    a.out[row * D + tid] = num / den;
    if (tid == 0 && a.lse != nullptr) a.lse[row] = (M + log2_hw(den)) * kLn2;
  }
}

template <int MODE, typename E, int D>
static hipError_t launch_p3(int G, const PartialArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)a.B * a.Hkv * a.nc)), block(kThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL((partial_kernel<MODE, E, D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((partial_kernel<MODE, E, D, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((partial_kernel<MODE, E, D, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((partial_kernel<MODE, E, D, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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

hipError_t launch_merge(int D, int B, const MergeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)B * a.Hq)), block(kThreads);
  if (D == 64) hipLaunchKernelGGL((merge_kernel<64>), grid, block, 0, s, a);
  else if (D == 128) hipLaunchKernelGGL((merge_kernel<128>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fdk
