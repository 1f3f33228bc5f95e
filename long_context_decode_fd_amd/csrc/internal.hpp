// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fdk {

enum Mode : int { kDense = 0, kPaged = 1, kUnified = 2 };

// Arguments of the split-KV partial kernel.  Scores are handled in units of
// the raw dot product q.k; `c_log2` = scale * log2(e) turns them into base-2
// exponents of the scaled score.
struct PartialArgs {
  const void* q;             // [B, Hq, D]
  const void* k;             // dense/unified: [B, Hkv, L, D]; paged: [P, Hkv, page, D]
  const void* v;
  float* o_part;             // [B, Hq, nc, D]   unnormalised chunk outputs
  float* ml_part;            // [B, Hq, nc, 2]   (m in log2 units, l)
  uint8_t* flags;            // unified only, [B, Hq, nc] or null
  const int32_t* block_table;  // paged only
  const int32_t* seq_lens;     // paged only
  int B, Hq, Hkv, L, chunk, nc;
  int page_shift, max_pages, num_pages, max_seq_len;
  float c_log2;
  float phi_raw;             // unified: phi / scale
  float flag_hi_raw;         // unified: (phi + margin_hi) / scale
  float flag_lo_raw;         // unified: (phi - margin_lo) / scale
};

struct MergeArgs {
  const float* o_part;
  const float* ml_part;
  float* out;                // [B, Hq, D]
  float* lse;                // [B, Hq] or null
  const int32_t* seq_lens;   // paged: chunk count per sequence; else null
  int Hq, nc, chunk, max_seq_len;
  // paged multi-row: the split is chunk * (*chunk_scale), the factor the
  // kernel chose on the device (values below 1 read as 1); else null
  const int32_t* chunk_scale;
};

hipError_t launch_partial(int mode, int is_bf16, int D, int G,
                          const PartialArgs& a, hipStream_t s);
hipError_t launch_merge(int D, int B, const MergeArgs& a, hipStream_t s);
// flags[i] = 1 where a chunk maximum m_i (ml[2 i], log2 units of the scaled
// score) lies above hi or below lo, else 0; n entries.
hipError_t launch_range_flags(const float* ml, uint8_t* flags, size_t n, float hi, float lo,
                              hipStream_t s);

struct FfdPackArgs {
  const uint16_t* k;   // bf16 [B, Hkv, Lcap, D]
  uint32_t* codes;     // [B, Hkv, Lcap, D/16]
  uint16_t* zs;        // [B, Hkv, Lcap, D/32, 2]
  int8_t* res;         // [B, Hkv, Lcap, D]
  uint16_t* rs;        // [B, Hkv, Lcap, D/32]
  int B, Hkv, Lcap, t_begin, t_end;
};
hipError_t launch_ffd_pack(int D, const FfdPackArgs& a, hipStream_t s);

struct FfdArgs {
  const uint16_t* q;   // bf16 [B, Hq, D]
  const uint32_t* codes;
  const uint16_t* zs;
  const int8_t* res;
  const uint16_t* rs;
  const uint16_t* v;   // bf16 [B, Hkv, L, D]
  float* o_part;
  float* ml_part;
  uint32_t* cand_mask; // [B, Hq, ceil(L/32)] or null
  float* pseudo_max;   // [B, Hq] or null (scaled units)
  float* anchor_max;   // workspace [B, Hq]: m^ in raw dot units
  int32_t* anchor_pos; // workspace [B, Hq]: j*
  int B, Hq, Hkv, L, chunk, nc, n_sink, n_local;
  float scale, c_log2, delta_raw;  // delta / scale
};
hipError_t launch_ffd(int D, int G, const FfdArgs& a, hipStream_t s);
// the wave-streamed FFD kernel (d = 128, G = 4 or 8), after the anchors
hipError_t launch_ffd_wave(int G, const FfdArgs& a, hipStream_t s);

// Multi-row decode: q [B, M, Hq, D] bf16, k/v [B, Hkv, L, D] bf16, partials
// for the rows (b, r, h) in the same layout as PartialArgs with M*Hq heads.
struct MultiArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o_part;
  float* ml_part;
  int B, M, Hq, Hkv, L, chunk, nc;
  float c_log2;
  // Paged caches (block_table != nullptr): k and v are pools [P, Hkv, page,
  // D], page = 2^page_shift >= 16; sequence b holds min(max(seq_lens[b], 0),
  // L) positions (L = the longest) through block_table[b * max_pages + i];
  // page ids are clamped to [0, num_pages).  A split (= chunk) covers at
  // most kMultiPagePids pages.
  const int32_t* block_table;
  const int32_t* seq_lens;
  int page_shift, max_pages, num_pages;
  // Paged: worker w's range of pages may start inside a chunk; that part's
  // partials go to row w * R + r of x_o [x_cap * R, D] and x_ml [x_cap * R,
  // 2] (R = G * M query rows) and x_meta[4 w ..] = (b, kv-head, chunk, 1)
  // (0 in the last entry when the range starts at a chunk start or is
  // empty), and a fix-up folds them into the chunks' partials.
  float* x_o;
  float* x_ml;
  int32_t* x_meta;
  int x_cap;
  // Paged: the kernel lengthens the split to chunk * F (F a power of two up
  // to 256, within the kernel's page-id buffer: kMultiPagePids pages, twice
  // that on the wave pair) as far as the workers keep their number, and
  // writes F here for the merge.
  int32_t* x_split;
};
constexpr int kMultiPagePids = 256;
// Workers of a paged multi-row call that get a slot for a part split off
// their first chunk (the workspace holds min(this, B * Hkv * nc) slots).
constexpr int kMultiWorkerCap = 2048;
hipError_t launch_multi(int D, const MultiArgs& a, hipStream_t s);
// Chunks per split for the multi-row kernels: the number of consecutive
// chunks of a row that one split covers, chosen so that the splits fill the
// device's wave slots with the fewest rounds (a.chunk and a.nc as called).
int multi_fold(int D, const MultiArgs& a);

// Compute units of the current device (cached per device).
int cu_count();

struct AppendArgs {
  const char* k_new;   // [B, Hkv, M, row]
  const char* v_new;
  char* k_dst;         // contiguous [B, Hkv, L_cap, row] or pool [P, Hkv, page, row]
  char* v_dst;
  const int32_t* block_table;  // paged only
  const int32_t* pos;          // paged only: first write position per sequence
  int B, Hkv, M, L_cap, t0, row_bytes, page_shift, max_pages, num_pages;
};
hipError_t launch_append(bool paged, const AppendArgs& a, hipStream_t s);

}  // namespace fdk
