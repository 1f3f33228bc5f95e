// Multi-row decode, one query tile (G*M <= 16 rows per kv-head), the
// dispatch between one tile and the wave pair, and the split length.
#include "multirow.hpp"

namespace fdk {

hipError_t launch_multi_pair(int D, const MultiArgs& a, hipStream_t s, int* workers);

size_t multi_pair_slots(int D);

// Splits of F consecutive chunks.  The latency estimate of the "Flash
// Decoding" explainer (section 2: each of the splits reads its share of the
// cache, then a merge whose cost grows with the number of splits) has its
// minimum once the splits fill the parallel hardware: more splits than the
// device runs at once only add partials to write and merge (two units of
// one wave cost it the same cache reads as one of twice the length, plus a
// partial of 4 (d + 2) bytes per query row).  F minimises the rounds of
// splits times their length, rows * ceil(nc / F) splits over `slots`
// concurrent ones; among equal makespans the largest F (fewest partials).
// Ragged last splits are the ragged chunks of the caller's chunking.
int multi_fold(int D, const MultiArgs& a) {
  const int R = (a.Hq / a.Hkv) * a.M;
  const size_t slots = R > 16 ? multi_pair_slots(D)
                              : (D == 64 ? multi_wave_slots<64>() : multi_wave_slots<128>());
  const size_t rows = (size_t)a.B * a.Hkv;
  const size_t units = rows * (size_t)a.nc;
  if (slots == 0 || units <= slots) return 1;
  // beyond twice the even share the makespan only grows
  const int hi = (int)std::min<size_t>((size_t)a.nc, 2 * ((units + slots - 1) / slots));
  int best = 1;
  size_t best_t = (size_t)-1;
  for (int f = 1; f <= hi; ++f) {
    const size_t n = rows * (size_t)((a.nc + f - 1) / f);
    const size_t t = ((n + slots - 1) / slots) * (size_t)f;
    if (t <= best_t) {
      best_t = t;
      best = f;
    }
  }
  return best;
}

// Paged calls: each part that a worker's range cut off a split's start
// (slot w, flagged in x_meta) is folded into that chunk's partials by the
// exact merge of two parts ("Flash Decoding" explainer, section 2):
// m = max(m1, m2), O = 2^(m1 - m) O1 + 2^(m2 - m) O2, l likewise (m in log2
// units).  A chunk has at most one such part, and its first part -- the
// previous worker's last -- sits in the chunk's own partials.  One wave per
// slot; a row neither part saw (m1 = m2 = -inf) keeps the empty partial.
template <int D>
__global__ __launch_bounds__(kWave) void multi_fixup_kernel(MultiArgs a, int workers) {
  const int w = (int)blockIdx.x;
  if (w >= workers) return;
  const int32_t* mt = a.x_meta + 4 * (size_t)w;
  if (mt[3] == 0) return;
  const int b = mt[0], kvh = mt[1], c = mt[2];
  const int G = a.Hq / a.Hkv, R = G * a.M;   // at most 32 rows
  constexpr int CPR = D / 4;                 // 16-byte pieces per row
  constexpr int NP = 32 * CPR / kWave;       // pieces of 32 rows per lane
  const int lane = (int)threadIdx.x;
  // every load first (one memory latency); rows past R read row R - 1 and
  // write nothing
  f32x4 o1[NP], o2[NP];
  f32x2 p1[NP], p2[NP];
  size_t prow[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int f = j * kWave + lane, r = min(f / CPR, R - 1), col = f % CPR;
    prow[j] = (((size_t)b * a.M + r / G) * a.Hq + (size_t)kvh * G + r % G) * a.nc + c;
    const size_t xrow = (size_t)w * R + r;
    o1[j] = reinterpret_cast<const f32x4*>(a.o_part + prow[j] * D)[col];
    o2[j] = reinterpret_cast<const f32x4*>(a.x_o + xrow * D)[col];
    p1[j] = *reinterpret_cast<const f32x2*>(a.ml_part + prow[j] * 2);
    p2[j] = *reinterpret_cast<const f32x2*>(a.x_ml + xrow * 2);
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int f = j * kWave + lane, col = f % CPR;
    const float M = fmaxf(p1[j].x, p2[j].x);
    if (f / CPR >= R || M == kNegInf) continue;   // padding, or a row neither part saw
    const float w1 = exp2_diff(p1[j].x, M), w2 = exp2_diff(p2[j].x, M);
    reinterpret_cast<f32x4*>(a.o_part + prow[j] * D)[col] =
        f32x4{fmaf(w1, o1[j].x, w2 * o2[j].x), fmaf(w1, o1[j].y, w2 * o2[j].y),
              fmaf(w1, o1[j].z, w2 * o2[j].z), fmaf(w1, o1[j].w, w2 * o2[j].w)};
    if (col == 0)
      *reinterpret_cast<f32x2*>(a.ml_part + prow[j] * 2) =
          f32x2{M, fmaf(w1, p1[j].y, w2 * p2[j].y)};
  }
}

hipError_t launch_multi(int D, const MultiArgs& a, hipStream_t s) {
  int workers = 0;
  hipError_t e = hipErrorInvalidValue;
  if ((a.Hq / a.Hkv) * a.M > 16) e = launch_multi_pair(D, a, s, &workers);
  else if (D == 64) e = launch_multi_d<64>(a, s, &workers);
  else if (D == 128) e = launch_multi_d<128>(a, s, &workers);
  if (e != hipSuccess || a.block_table == nullptr) return e;
  workers = std::min(workers, a.x_cap);
  if (workers <= 0) return hipSuccess;
  if (D == 64)
    hipLaunchKernelGGL((multi_fixup_kernel<64>), dim3((unsigned)workers), dim3(kWave), 0, s, a, workers);
  else
    hipLaunchKernelGGL((multi_fixup_kernel<128>), dim3((unsigned)workers), dim3(kWave), 0, s, a, workers);
  return hipGetLastError();
}

}  // namespace fdk
