// Multi-row decode, one query tile (G*M <= 16 rows per kv-head), the
// dispatch between one tile and the wave pair, and the split length.
#include "multirow.hpp"

namespace fdk {

hipError_t launch_multi_pair(int D, const MultiArgs& a, hipStream_t s);

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

hipError_t launch_multi(int D, const MultiArgs& a, hipStream_t s) {
  if ((a.Hq / a.Hkv) * a.M > 16) return launch_multi_pair(D, a, s);
  if (D == 64) return launch_multi_d<64>(a, s);
  if (D == 128) return launch_multi_d<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fdk
