// C ABI entry points (see include/fd.h): argument validation, workspace
// sizing, kernel dispatch.  Nothing here allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>

#include "../../include/fd.h"
#include "internal.hpp"

// Chunk partials of fd_decode_attn_noalloc: a buffer owned by the library,
// one copy on every device the library runs on (held until the process
// ends).  Host code never uses this name as an address: the device address
// of each device's copy comes from hipGetSymbolAddress (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[FD_NOALLOC_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return FD_OK;
}

// A caller of the C ABI may pass any int as fd_dtype_t; in C++ an enum
// value outside its enumerators' range is undefined, so the argument is
// never read as an enum before this check: its integer representation is.
int check_dtype(const fd_dtype_t* dt) {
  int code;
  memcpy(&code, dt, sizeof code);
  if (code != FD_F32 && code != FD_BF16) return fail(FD_ERR_ARG, "unknown dtype %d", code);
  return FD_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_heads(int B, int Hq, int Hkv, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
    return fail(FD_ERR_ARG, "B=%d Hq=%d Hkv=%d d=%d must be positive", B, Hq, Hkv, d);
  if (Hq % Hkv != 0) return fail(FD_ERR_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (d != 64 && d != 128) return fail(FD_ERR_UNSUPPORTED, "d=%d not in {64,128}", d);
  return FD_OK;
}

// Group sizes of the single-query vector kernels (paged, fixed maximum, FFD
// and the dense path's fast case).
bool vector_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

int check_vector_group(int G) {
  if (!vector_group(G))
    return fail(FD_ERR_UNSUPPORTED, "group size Hq/Hkv=%d not in {1,2,4,8}", G);
  return FD_OK;
}

// Dense paths: M query tokens per sequence.  Every case the vector kernel
// (one token, G in {1,2,4,8}, bf16 or fp32) does not take runs on the
// matrix-core kernels, which take bf16 and up to 32 query rows (G * M) per
// kv-head.
bool matrix_needed(int G, int M) { return M > 1 || !vector_group(G); }

int check_dense_group(fd_dtype_t dt, int G, int M) {
  if (!matrix_needed(G, M)) return FD_OK;
  if ((long long)G * M > 32)
    return fail(FD_ERR_UNSUPPORTED, "G*M=%lld query rows per kv-head exceed 32",
                (long long)G * M);
  if (dt != FD_BF16)
    return fail(FD_ERR_UNSUPPORTED, "several query tokens, or a group size outside "
                                    "{1,2,4,8}, need bf16 inputs");
  return FD_OK;
}

// Paged cache arguments of both paged entry points; *shift = log2(page).
int check_pages(int chunk, int page_size, int min_page, int max_pages_per_seq, int num_pages,
                int max_seq_len, int* shift) {
  if (page_size < min_page || page_size > 1024 || (page_size & (page_size - 1)) != 0)
    return fail(FD_ERR_ARG, "page_size=%d must be a power of two in [%d, 1024]", page_size,
                min_page);
  if (chunk % page_size != 0)
    return fail(FD_ERR_ARG, "chunk=%d must be a multiple of page_size=%d", chunk, page_size);
  if (max_pages_per_seq <= 0 || num_pages <= 0)
    return fail(FD_ERR_ARG, "max_pages_per_seq and num_pages must be positive");
  if (max_seq_len < 0 || (long long)max_seq_len > (long long)max_pages_per_seq * page_size)
    return fail(FD_ERR_ARG, "max_seq_len=%d outside [0, max_pages_per_seq*page_size]",
                max_seq_len);
  *shift = 0;
  while ((1 << *shift) < page_size) ++*shift;
  return FD_OK;
}

int check_chunk(int chunk) {
  if (chunk <= 0 || chunk % 16 != 0 || chunk > 65536)
    return fail(FD_ERR_ARG, "chunk=%d must be a positive multiple of 16 <= 65536", chunk);
  return FD_OK;
}

int check_scale(float scale) {
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(FD_ERR_ARG, "scale must be finite and positive");
  return FD_OK;
}

// The kernels number units (sequence, kv-head, chunk) and rows of queries
// with 32-bit integers.
int check_units(int B, int H, int nc) {
  if ((long long)B * H * nc > 0x7FFFFFFFLL || (long long)B * H > 0x7FFFFFFFLL / 2)
    return fail(FD_ERR_UNSUPPORTED, "B=%d x %d heads x %d chunks exceeds 32-bit unit indices",
                B, H, nc);
  return FD_OK;
}

int n_chunks_of(int L, int chunk) { return (int)(((long long)L + chunk - 1) / chunk); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Partials workspace: O [B*Hq*nc*d] fp32, then (m, l) [B*Hq*nc*2] fp32.
size_t partial_bytes(int B, int Hq, int nc, int d) {
  const size_t rows = (size_t)B * Hq * nc;
  const size_t n = align256(rows * d * sizeof(float)) + align256(rows * 2 * sizeof(float));
  return n > 256 ? n : 256;
}

// Paged multi-row calls: worker slots for the parts split off a chunk's
// start (at most one per worker, and never more workers than units).
int multi_worker_slots(int B, int Hkv, int nc) {
  const long long units = (long long)B * Hkv * nc;
  return (int)std::min<long long>(std::max<long long>(units, 1), fdk::kMultiWorkerCap);
}

size_t multi_worker_bytes(int B, int Hkv, int nc, int R, int d) {
  const size_t slots = (size_t)multi_worker_slots(B, Hkv, nc);
  return align256(slots * R * d * sizeof(float)) + align256(slots * R * 2 * sizeof(float)) +
         align256(slots * 4 * sizeof(int32_t)) + 256;
}

int workspace_gate(void* ws, size_t* ws_bytes, size_t need) {
  if (ws_bytes == nullptr) return fail(FD_ERR_ARG, "ws_bytes is NULL");
  if (ws == nullptr) {
    *ws_bytes = need;
    return FD_OK;
  }
  if (((uintptr_t)ws & 255) != 0) return fail(FD_ERR_ARG, "ws must be 256-byte aligned");
  if (*ws_bytes < need)
    return fail(FD_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", *ws_bytes, need);
  return FD_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

void split_ws(void* ws, int B, int Hq, int nc, int d, float** o_part, float** ml_part) {
  const size_t rows = (size_t)B * Hq * nc;
  *o_part = reinterpret_cast<float*>(ws);
  *ml_part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                      align256(rows * d * sizeof(float)));
}

// Split for a full call on the vector kernel.  A call whose (sequence,
// kv-head, chunk) units are fewer than MI355X's 1,024 SIMDs (256 compute
// units x 4) would leave SIMDs without a share of the cache, so the split
// halves (down to 32 positions, staying a multiple of 16 and of `unit`, the
// page of a paged cache) until the units reach 1,024; the merge takes blocks
// of any length ("Flash Decoding" explainer, section 2), so only fp32
// rounding changes.  L is the longest sequence.  A fixed device model keeps
// the workspace size a pure function of the arguments.
constexpr long long kSimdUnits = 1024;

int full_call_split(int B, int Hkv, int L, int chunk, int unit = 16) {
  int split = chunk;
  while ((long long)B * Hkv * n_chunks_of(L, split) < kSimdUnits && split % 32 == 0 &&
         split / 2 >= 32 && (split / 2) % unit == 0)
    split /= 2;
  return split;
}

// The matrix-core kernels also take, by choice, bf16 single-token calls
// with G = 8 once they have at least 1,024 (sequence, kv-head, chunk) units
// (L: the longest sequence): eight query heads per lane group leave the
// vector kernel issue-bound (B 8, Hkv 8, L 32768, d 128: 240.7 us, 56 % of
// 8 TB/s) where the matrix cores take the products (161.6 us, 83 %); d 64:
// 126.8 -> 100.6 us.  Shorter calls keep the vector kernel and its shorter
// splits (B 1, L 32768: 39.4 against 44.1 us).
bool matrix_path(fd_dtype_t dt, int G, int M, int B, int Hkv, int L, int chunk) {
  if (matrix_needed(G, M)) return true;
  return dt == FD_BF16 && G == 8 && (long long)B * Hkv * n_chunks_of(L, chunk) >= kSimdUnits;
}

// Enqueue the partial kernel and (when out != NULL) the merge.
int run_split_kv(int mode, fd_dtype_t dt, const void* q, const void* k, const void* v,
                 float* out, float* lse, int B, int Hq, int Hkv, int L, int d,
                 float scale, int chunk, int nc, fdk::PartialArgs pa, void* ws,
                 const int32_t* seq_lens, int max_seq_len, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float *o_part, *ml_part;
  split_ws(ws, B, Hq, nc, d, &o_part, &ml_part);
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.o_part = o_part;
  pa.ml_part = ml_part;
  pa.B = B;
  pa.Hq = Hq;
  pa.Hkv = Hkv;
  pa.L = L;
  pa.chunk = chunk;
  pa.nc = nc;
  pa.c_log2 = (float)((double)scale * 1.4426950408889634);
  if (nc > 0) {
    hipError_t e = fdk::launch_partial(mode, dt == FD_BF16, d, Hq / Hkv, pa, s);
    if (e != hipSuccess) return hip_status(e, "partial kernel launch");
  }
  if (out == nullptr) return ok();
  fdk::MergeArgs ma{o_part, ml_part, out, lse, seq_lens, Hq, nc, chunk, max_seq_len, nullptr};
  return hip_status(fdk::launch_merge(d, B, ma, s), "merge kernel launch");
}

// Enqueue the matrix-core kernel for M tokens of G*M <= 32 query rows per
// kv-head and (when out != NULL) the merge.  fold: splits may cover several
// consecutive chunks (fewer partials when the chunks outnumber the device's
// wave slots); without it every chunk gets its own partial, as
// fd_decode_attn_partials promises.  The workspace sized for nc chunks holds
// either.
int run_multi(const void* q, const void* k, const void* v, float* out, float* lse, int B,
              int M, int Hq, int Hkv, int L, int d, float scale, int chunk, int nc, void* ws,
              bool fold, void* stream, const fdk::MultiArgs* paged = nullptr) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  fdk::MultiArgs ma{q, k, v, nullptr, nullptr, B, M, Hq, Hkv, L, chunk, nc,
                    (float)((double)scale * 1.4426950408889634), nullptr, nullptr, 0, 0, 0,
                    nullptr, nullptr, nullptr, 0, nullptr};
  if (paged != nullptr) {
    ma.block_table = paged->block_table;
    ma.seq_lens = paged->seq_lens;
    ma.page_shift = paged->page_shift;
    ma.max_pages = paged->max_pages;
    ma.num_pages = paged->num_pages;
  } else if (nc > 0) {
    // paged calls keep the caller's chunk as the split (the lengths that
    // would decide a longer one live on the device; the kernels split the
    // pages that hold positions evenly over the workers)
    const int F = fold ? fdk::multi_fold(d, ma) : 1;
    const long long split = (long long)chunk * F;
    ma.chunk = split > L ? L : (int)split;
    ma.nc = n_chunks_of(L, ma.chunk);
  }
  split_ws(ws, B, M * Hq, ma.nc, d, &ma.o_part, &ma.ml_part);
  if (paged != nullptr) {
    const int R = (Hq / Hkv) * M;
    ma.x_cap = multi_worker_slots(B, Hkv, ma.nc);
    char* x = reinterpret_cast<char*>(ws) + partial_bytes(B, M * Hq, ma.nc, d);
    ma.x_o = reinterpret_cast<float*>(x);
    x += align256((size_t)ma.x_cap * R * d * sizeof(float));
    ma.x_ml = reinterpret_cast<float*>(x);
    x += align256((size_t)ma.x_cap * R * 2 * sizeof(float));
    ma.x_meta = reinterpret_cast<int32_t*>(x);
    x += align256((size_t)ma.x_cap * 4 * sizeof(int32_t));
    ma.x_split = reinterpret_cast<int32_t*>(x);
  }
  if (ma.nc > 0) {
    hipError_t e = fdk::launch_multi(d, ma, s);
    if (e != hipSuccess) return hip_status(e, "multi-row kernel launch");
  }
  if (out == nullptr) return ok();
  fdk::MergeArgs mg{ma.o_part, ma.ml_part, out, lse, ma.seq_lens, M * Hq, ma.nc, ma.chunk, L,
                    ma.x_split};
  return hip_status(fdk::launch_merge(d, B, mg, s), "merge kernel launch");
}

// Device address of `scratch` on each device, resolved once per device
// with that device current (the first fd_decode_attn_noalloc call there).
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FD_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(FD_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FD_OK;
}

}  // namespace

extern "C" {

const char* fd_last_error(void) { return g_err.c_str(); }

int fd_abi_version(void) { return 1; }

int fd_decode_attn(fd_dtype_t dt, const void* q, const void* k, const void* v, float* out,
                   float* lse, int B, int Hq, int Hkv, int L, int d, float scale, int chunk,
                   void* ws, size_t* ws_bytes, void* stream) {
  if (int e = check_dtype(&dt)) return e;
  if (int e = check_heads(B, Hq, Hkv, d)) return e;
  if (int e = check_dense_group(dt, Hq / Hkv, 1)) return e;
  if (L <= 0) return fail(FD_ERR_ARG, "L=%d must be positive", L);
  if (int e = check_chunk(chunk)) return e;
  if (int e = check_scale(scale)) return e;
  const int nc = n_chunks_of(L, chunk);
  if (int e = check_units(B, Hq, nc)) return e;
  const bool matrix = matrix_path(dt, Hq / Hkv, 1, B, Hkv, L, chunk);
  const int split = matrix ? chunk : full_call_split(B, Hkv, L, chunk);
  const int ns = n_chunks_of(L, split);
  if (int e = check_units(B, Hq, ns)) return e;
  if (int e = workspace_gate(ws, ws_bytes, partial_bytes(B, Hq, ns, d))) return e;
  if (ws == nullptr) return ok();
  if (!q || !k || !v || !out) return fail(FD_ERR_ARG, "q, k, v and out must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(FD_ERR_ARG, "q, k, v and out must be 16-byte aligned");
  if (matrix)
    return run_multi(q, k, v, out, lse, B, 1, Hq, Hkv, L, d, scale, chunk, nc, ws, true, stream);
  fdk::PartialArgs pa{};
  return run_split_kv(fdk::kDense, dt, q, k, v, out, lse, B, Hq, Hkv, L, d, scale, split, ns,
                      pa, ws, nullptr, L, stream);
}

int fd_decode_attn_noalloc(fd_dtype_t dt, const void* q, const void* k, const void* v,
                           float* out, float* lse, int B, int Hq, int Hkv, int L, int d,
                           float scale, int chunk, void* stream) {
  if (int e = check_dtype(&dt)) return e;
  if (int e = check_heads(B, Hq, Hkv, d)) return e;
  if (int e = check_dense_group(dt, Hq / Hkv, 1)) return e;
  if (L <= 0) return fail(FD_ERR_ARG, "L=%d must be positive", L);
  if (int e = check_chunk(chunk)) return e;
  if (int e = check_scale(scale)) return e;
  const int nc = n_chunks_of(L, chunk);
  if (int e = check_units(B, Hq, nc)) return e;
  const bool matrix = matrix_path(dt, Hq / Hkv, 1, B, Hkv, L, chunk);
  const int split = matrix ? chunk : full_call_split(B, Hkv, L, chunk);
  const int ns = n_chunks_of(L, split);
  if (int e = check_units(B, Hq, ns)) return e;
  const size_t need = partial_bytes(B, Hq, ns, d);
  if (need > (size_t)FD_NOALLOC_BYTES)
    return fail(FD_ERR_WORKSPACE,
                "%zu bytes of chunk partials exceed the library's %zu-byte buffer "
                "(use fd_decode_attn with a workspace, or longer chunks)",
                need, (size_t)FD_NOALLOC_BYTES);
  if (!q || !k || !v || !out) return fail(FD_ERR_ARG, "q, k, v and out must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(FD_ERR_ARG, "q, k, v and out must be 16-byte aligned");
  void* ws = nullptr;
  if (int e = scratch_ptr(&ws)) return e;
  if (matrix)
    return run_multi(q, k, v, out, lse, B, 1, Hq, Hkv, L, d, scale, chunk, nc, ws, true, stream);
  fdk::PartialArgs pa{};
  return run_split_kv(fdk::kDense, dt, q, k, v, out, lse, B, Hq, Hkv, L, d, scale, split, ns,
                      pa, ws, nullptr, L, stream);
}

int fd_decode_attn_partials(fd_dtype_t dt, const void* q, const void* k, const void* v,
                            int B, int Hq, int Hkv, int L, int d, float scale, int chunk,
                            void* ws, size_t* ws_bytes, void* stream) {
  if (int e = check_dtype(&dt)) return e;
  if (int e = check_heads(B, Hq, Hkv, d)) return e;
  if (int e = check_dense_group(dt, Hq / Hkv, 1)) return e;
  if (L <= 0) return fail(FD_ERR_ARG, "L=%d must be positive", L);
  if (int e = check_chunk(chunk)) return e;
  if (int e = check_scale(scale)) return e;
  const int nc = n_chunks_of(L, chunk);
  if (int e = check_units(B, Hq, nc)) return e;
  if (int e = workspace_gate(ws, ws_bytes, partial_bytes(B, Hq, nc, d))) return e;
  if (ws == nullptr) return ok();
  if (!q || !k || !v) return fail(FD_ERR_ARG, "q, k and v must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(FD_ERR_ARG, "q, k and v must be 16-byte aligned");
  if (matrix_path(dt, Hq / Hkv, 1, B, Hkv, L, chunk))
    return run_multi(q, k, v, nullptr, nullptr, B, 1, Hq, Hkv, L, d, scale, chunk, nc, ws,
                     false, stream);
  fdk::PartialArgs pa{};
  return run_split_kv(fdk::kDense, dt, q, k, v, nullptr, nullptr, B, Hq, Hkv, L, d, scale,
                      chunk, nc, pa, ws, nullptr, L, stream);
}

int fd_merge_partials(const float* o_part, const float* ml_part, float* out, float* lse,
                      int B, int Hq, int n_chunks, int d, void* stream) {
  if (B <= 0 || Hq <= 0 || n_chunks <= 0)
    return fail(FD_ERR_ARG, "B=%d Hq=%d n_chunks=%d must be positive", B, Hq, n_chunks);
  if (d != 64 && d != 128) return fail(FD_ERR_UNSUPPORTED, "d=%d not in {64,128}", d);
  if (int e = check_units(B, Hq, n_chunks)) return e;
  if (!o_part || !ml_part || !out) return fail(FD_ERR_ARG, "o_part, ml_part, out NULL");
  if (!aligned16(o_part) || !aligned16(ml_part) || !aligned16(out))
    return fail(FD_ERR_ARG, "o_part, ml_part and out must be 16-byte aligned");
  fdk::MergeArgs ma{o_part, ml_part, out, lse, nullptr, Hq, n_chunks, 1, 0, nullptr};
  return hip_status(fdk::launch_merge(d, B, ma, reinterpret_cast<hipStream_t>(stream)),
                    "merge kernel launch");
}

int fd_decode_attn_paged(fd_dtype_t dt, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_table,
                         const int32_t* seq_lens, float* out, float* lse, int B, int Hq,
                         int Hkv, int d, int page_size, int max_pages_per_seq,
                         int num_pages, int max_seq_len, float scale, int chunk, void* ws,
                         size_t* ws_bytes, void* stream) {
  if (int e = check_dtype(&dt)) return e;
  if (int e = check_heads(B, Hq, Hkv, d)) return e;
  if (int e = check_vector_group(Hq / Hkv)) return e;
  if (int e = check_chunk(chunk)) return e;
  if (int e = check_scale(scale)) return e;
  int shift = 0;
  if (int e = check_pages(chunk, page_size, 8, max_pages_per_seq, num_pages, max_seq_len, &shift))
    return e;
  if (chunk / page_size > 1024)
    return fail(FD_ERR_UNSUPPORTED, "chunk/page_size=%d exceeds 1024", chunk / page_size);
  // bf16 with G = 8 on a long call: the matrix-core kernel of the multi-row
  // entry point with one token (q [B, Hq, d] is q [B, 1, Hq, d])
  if (matrix_path(dt, Hq / Hkv, 1, B, Hkv, max_seq_len, chunk) && page_size >= 16 &&
      chunk / page_size <= fdk::kMultiPagePids)
    return fd_decode_attn_multi_paged(dt, q, k_pool, v_pool, block_table, seq_lens, out, lse, B,
                                      1, Hq, Hkv, d, page_size, max_pages_per_seq, num_pages,
                                      max_seq_len, scale, chunk, ws, ws_bytes, stream);
  const int split = full_call_split(B, Hkv, max_seq_len, chunk, page_size);
  const int nc = n_chunks_of(max_seq_len, split);
  if (int e = check_units(B, Hq, nc)) return e;
  if (int e = workspace_gate(ws, ws_bytes, partial_bytes(B, Hq, nc, d))) return e;
  if (ws == nullptr) return ok();
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !out)
    return fail(FD_ERR_ARG, "q, pools, block_table, seq_lens and out must not be NULL");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return fail(FD_ERR_ARG, "q, pools and out must be 16-byte aligned");
  fdk::PartialArgs pa{};
  pa.block_table = block_table;
  pa.seq_lens = seq_lens;
  pa.page_shift = shift;
  pa.max_pages = max_pages_per_seq;
  pa.num_pages = num_pages;
  pa.max_seq_len = max_seq_len;
  return run_split_kv(fdk::kPaged, dt, q, k_pool, v_pool, out, lse, B, Hq, Hkv, 0, d, scale,
                      split, nc, pa, ws, seq_lens, max_seq_len, stream);
}

int fd_decode_attn_unified_max(fd_dtype_t dt, const void* q, const void* k, const void* v,
                               float* out, float* lse, int B, int Hq, int Hkv, int L, int d,
                               float scale, int chunk, float phi, float margin_hi,
                               float margin_lo, uint8_t* chunk_flags, void* ws,
                               size_t* ws_bytes, void* stream) {
  if (int e = check_dtype(&dt)) return e;
  if (int e = check_heads(B, Hq, Hkv, d)) return e;
  if (int e = check_vector_group(Hq / Hkv)) return e;
  if (L <= 0) return fail(FD_ERR_ARG, "L=%d must be positive", L);
  if (int e = check_chunk(chunk)) return e;
  if (int e = check_scale(scale)) return e;
  if (!isfinite(phi)) return fail(FD_ERR_ARG, "phi must be finite");
  if (!(margin_hi >= 0.f && margin_hi <= 60.f) || !(margin_lo >= 0.f && margin_lo <= 60.f))
    return fail(FD_ERR_ARG, "margins must lie in [0, 60] (exp(60) bounds the fp32 sums)");
  const int nc = n_chunks_of(L, chunk);
  if (int e = check_units(B, Hq, nc)) return e;
  if (int e = workspace_gate(ws, ws_bytes, partial_bytes(B, Hq, nc, d))) return e;
  if (ws == nullptr) return ok();
  if (!q || !k || !v || !out) return fail(FD_ERR_ARG, "q, k, v and out must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(FD_ERR_ARG, "q, k, v and out must be 16-byte aligned");
  if (matrix_path(dt, Hq / Hkv, 1, B, Hkv, L, chunk)) {
    // bf16 with G = 8 on a long call: every chunk with its own maximum on
    // the matrix-core kernel (exact; the fixed maximum saves no work there),
    // and the range flags from the chunks' maxima, kept per chunk (m in
    // log2 units of the scaled score: the bounds times log2 e)
    if (int e = run_multi(q, k, v, out, lse, B, 1, Hq, Hkv, L, d, scale, chunk, nc, ws, false,
                          stream))
      return e;
    if (chunk_flags == nullptr) return ok();
    float *o_part, *ml_part;
    split_ws(ws, B, Hq, nc, d, &o_part, &ml_part);
    const double l2e = 1.4426950408889634;
    return hip_status(
        fdk::launch_range_flags(ml_part, chunk_flags, (size_t)B * Hq * nc,
                                (float)(((double)phi + margin_hi) * l2e),
                                (float)(((double)phi - margin_lo) * l2e),
                                reinterpret_cast<hipStream_t>(stream)),
        "range flags launch");
  }
  fdk::PartialArgs pa{};
  pa.flags = chunk_flags;
  pa.phi_raw = (float)((double)phi / (double)scale);
  pa.flag_hi_raw = (float)(((double)phi + margin_hi) / (double)scale);
  pa.flag_lo_raw = (float)(((double)phi - margin_lo) / (double)scale);
  return run_split_kv(fdk::kUnified, dt, q, k, v, out, lse, B, Hq, Hkv, L, d, scale, chunk,
                      nc, pa, ws, nullptr, L, stream);
}

int fd_decode_attn_multi(fd_dtype_t dt, const void* q, const void* k, const void* v,
                         float* out, float* lse, int B, int M, int Hq, int Hkv, int L, int d,
                         float scale, int chunk, void* ws, size_t* ws_bytes, void* stream) {
  if (int e = check_dtype(&dt)) return e;
  if (int e = check_heads(B, Hq, Hkv, d)) return e;
  if (M <= 0) return fail(FD_ERR_ARG, "M=%d must be positive", M);
  if (L < M) return fail(FD_ERR_ARG, "L=%d must be at least M=%d", L, M);
  if (int e = check_chunk(chunk)) return e;
  if (int e = check_scale(scale)) return e;
  if (int e = check_dense_group(dt, Hq / Hkv, M)) return e;
  const int nc = n_chunks_of(L, chunk);
  if (int e = check_units(B, M * Hq, nc)) return e;
  const bool matrix = matrix_path(dt, Hq / Hkv, M, B, Hkv, L, chunk);
  const int split = matrix ? chunk : full_call_split(B, Hkv, L, chunk);
  const int ns = n_chunks_of(L, split);
  if (int e = check_units(B, M * Hq, ns)) return e;
  if (int e = workspace_gate(ws, ws_bytes, partial_bytes(B, M * Hq, ns, d))) return e;
  if (ws == nullptr) return ok();
  if (!q || !k || !v || !out) return fail(FD_ERR_ARG, "q, k, v and out must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(FD_ERR_ARG, "q, k, v and out must be 16-byte aligned");
  if (!matrix) {
    // one query row per head of a group the vector kernel takes
    // (q [B, 1, Hq, d] is q [B, Hq, d]): fd_decode_attn
    fdk::PartialArgs pa{};
    return run_split_kv(fdk::kDense, dt, q, k, v, out, lse, B, Hq, Hkv, L, d, scale, split, ns,
                        pa, ws, nullptr, L, stream);
  }
  return run_multi(q, k, v, out, lse, B, M, Hq, Hkv, L, d, scale, chunk, nc, ws, true, stream);
}

int fd_decode_attn_multi_paged(fd_dtype_t dt, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, float* out, float* lse, int B, int M,
                               int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                               int num_pages, int max_seq_len, float scale, int chunk, void* ws,
                               size_t* ws_bytes, void* stream) {
  if (int e = check_dtype(&dt)) return e;
  if (int e = check_heads(B, Hq, Hkv, d)) return e;
  if (M <= 0) return fail(FD_ERR_ARG, "M=%d must be positive", M);
  if (int e = check_dense_group(dt, Hq / Hkv, M)) return e;
  if (int e = check_chunk(chunk)) return e;
  if (int e = check_scale(scale)) return e;
  int shift = 0;
  if (int e = check_pages(chunk, page_size, 8, max_pages_per_seq, num_pages, max_seq_len, &shift))
    return e;
  // the optional matrix-core case (G = 8) only where its page limits hold
  const bool matrix = matrix_needed(Hq / Hkv, M) ||
                      (matrix_path(dt, Hq / Hkv, M, B, Hkv, max_seq_len, chunk) &&
                       page_size >= 16 && chunk / page_size <= fdk::kMultiPagePids);
  if (matrix && page_size < 16)
    return fail(FD_ERR_UNSUPPORTED, "page_size=%d: the matrix-core kernels take pages of 16 "
                                    "positions or more", page_size);
  if (chunk / page_size > (matrix ? fdk::kMultiPagePids : 1024))
    return fail(FD_ERR_UNSUPPORTED, "chunk/page_size=%d exceeds %d", chunk / page_size,
                matrix ? fdk::kMultiPagePids : 1024);
  const int split = matrix ? chunk : full_call_split(B, Hkv, max_seq_len, chunk, page_size);
  const int nc = n_chunks_of(max_seq_len, split);
  if (int e = check_units(B, M * Hq, nc)) return e;
  const int R = (Hq / Hkv) * M;
  const size_t need = partial_bytes(B, M * Hq, nc, d) +
                      (matrix ? multi_worker_bytes(B, Hkv, nc, R, d) : 0);
  if (int e = workspace_gate(ws, ws_bytes, need)) return e;
  if (ws == nullptr) return ok();
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !out)
    return fail(FD_ERR_ARG, "q, pools, block_table, seq_lens and out must not be NULL");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return fail(FD_ERR_ARG, "q, pools and out must be 16-byte aligned");
  if (!matrix) {
    // one token, a group the vector kernel takes: the paged single-query path
    fdk::PartialArgs pa{};
    pa.block_table = block_table;
    pa.seq_lens = seq_lens;
    pa.page_shift = shift;
    pa.max_pages = max_pages_per_seq;
    pa.num_pages = num_pages;
    pa.max_seq_len = max_seq_len;
    return run_split_kv(fdk::kPaged, dt, q, k_pool, v_pool, out, lse, B, Hq, Hkv, 0, d, scale,
                        split, nc, pa, ws, seq_lens, max_seq_len, stream);
  }
  fdk::MultiArgs pg{};
  pg.block_table = block_table;
  pg.seq_lens = seq_lens;
  pg.page_shift = shift;
  pg.max_pages = max_pages_per_seq;
  pg.num_pages = num_pages;
  return run_multi(q, k_pool, v_pool, out, lse, B, M, Hq, Hkv, max_seq_len, d, scale, chunk, nc,
                   ws, true, stream, &pg);
}

int fd_kv_append(fd_dtype_t dt, const void* k_new, const void* v_new, void* k_cache,
                 void* v_cache, int B, int Hkv, int M, int L_cap, int d, int t, void* stream) {
  if (int e = check_dtype(&dt)) return e;
  if (B <= 0 || Hkv <= 0 || M <= 0 || L_cap <= 0)
    return fail(FD_ERR_ARG, "B=%d Hkv=%d M=%d L_cap=%d must be positive", B, Hkv, M, L_cap);
  if (d != 64 && d != 128) return fail(FD_ERR_UNSUPPORTED, "d=%d not in {64,128}", d);
  if (t < 0 || t > L_cap - M)
    return fail(FD_ERR_ARG, "rows t=%d .. t+M-1=%d outside the cache of %d", t, t + M - 1, L_cap);
  if (!k_new || !v_new || !k_cache || !v_cache) return fail(FD_ERR_ARG, "NULL array");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(FD_ERR_ARG, "arrays must be 16-byte aligned");
  fdk::AppendArgs a{};
  a.k_new = static_cast<const char*>(k_new);
  a.v_new = static_cast<const char*>(v_new);
  a.k_dst = static_cast<char*>(k_cache);
  a.v_dst = static_cast<char*>(v_cache);
  a.B = B; a.Hkv = Hkv; a.M = M; a.L_cap = L_cap; a.t0 = t;
  a.row_bytes = d * (dt == FD_BF16 ? 2 : 4);
  return hip_status(fdk::launch_append(false, a, reinterpret_cast<hipStream_t>(stream)),
                    "append kernel launch");
}

int fd_kv_append_paged(fd_dtype_t dt, const void* k_new, const void* v_new, void* k_pool,
                       void* v_pool, const int32_t* block_table, const int32_t* pos, int B,
                       int Hkv, int M, int d, int page_size, int max_pages_per_seq,
                       int num_pages, void* stream) {
  if (int e = check_dtype(&dt)) return e;
  if (B <= 0 || Hkv <= 0 || M <= 0 || max_pages_per_seq <= 0 || num_pages <= 0)
    return fail(FD_ERR_ARG, "B=%d Hkv=%d M=%d max_pages=%d num_pages=%d must be positive", B,
                Hkv, M, max_pages_per_seq, num_pages);
  if (d != 64 && d != 128) return fail(FD_ERR_UNSUPPORTED, "d=%d not in {64,128}", d);
  if (page_size < 8 || page_size > 1024 || (page_size & (page_size - 1)) != 0)
    return fail(FD_ERR_ARG, "page_size=%d must be a power of two in [8, 1024]", page_size);
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !pos)
    return fail(FD_ERR_ARG, "NULL array");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(FD_ERR_ARG, "arrays must be 16-byte aligned");
  fdk::AppendArgs a{};
  a.k_new = static_cast<const char*>(k_new);
  a.v_new = static_cast<const char*>(v_new);
  a.k_dst = static_cast<char*>(k_pool);
  a.v_dst = static_cast<char*>(v_pool);
  a.block_table = block_table;
  a.pos = pos;
  a.B = B; a.Hkv = Hkv; a.M = M;
  a.row_bytes = d * (dt == FD_BF16 ? 2 : 4);
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  a.page_shift = shift;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  return hip_status(fdk::launch_append(true, a, reinterpret_cast<hipStream_t>(stream)),
                    "paged append kernel launch");
}

int fd_ffd_pack(const void* k, uint32_t* codes, uint16_t* zs, int8_t* res, uint16_t* rs,
                int B, int Hkv, int L_cap, int d, int t_begin, int t_end, void* stream) {
  if (B <= 0 || Hkv <= 0 || L_cap <= 0)
    return fail(FD_ERR_ARG, "B=%d Hkv=%d L_cap=%d must be positive", B, Hkv, L_cap);
  if (d != 64 && d != 128) return fail(FD_ERR_UNSUPPORTED, "d=%d not in {64,128}", d);
  if (t_begin < 0 || t_begin > t_end || t_end > L_cap)
    return fail(FD_ERR_ARG, "need 0 <= t_begin=%d <= t_end=%d <= L_cap=%d", t_begin, t_end,
                L_cap);
  if (!k || !codes || !zs || !res || !rs) return fail(FD_ERR_ARG, "NULL array");
  if (!aligned16(k) || !aligned16(codes) || !aligned16(res) || ((uintptr_t)zs & 3) != 0)
    return fail(FD_ERR_ARG, "k, codes and res must be 16-byte and zs 4-byte aligned");
  if (t_begin == t_end) return ok();
  fdk::FfdPackArgs pa{reinterpret_cast<const uint16_t*>(k), codes, zs, res, rs, B, Hkv, L_cap,
                      t_begin, t_end};
  return hip_status(fdk::launch_ffd_pack(d, pa, reinterpret_cast<hipStream_t>(stream)),
                    "pack kernel launch");
}

int fd_ffd_sparse_decode(const void* q, const uint32_t* codes, const uint16_t* zs,
                         const int8_t* res, const uint16_t* rs, const void* v, float* out,
                         float* lse, int B, int Hq, int Hkv, int L, int d, float scale,
                         float delta, int n_sink, int n_local, int chunk, uint32_t* cand_mask,
                         float* pseudo_max, void* ws, size_t* ws_bytes, void* stream) {
  if (int e = check_heads(B, Hq, Hkv, d)) return e;
  if (int e = check_vector_group(Hq / Hkv)) return e;
  if (L <= 0) return fail(FD_ERR_ARG, "L=%d must be positive", L);
  if (int e = check_chunk(chunk)) return e;
  {
    // the kernel keeps a chunk's scan scores, masks and candidate list in
    // LDS: (4 G + 3) bytes per position, at most 38 KiB with these limits
    const int cmax = (Hq / Hkv) >= 8 ? 1024 : 2048;
    if (chunk % 32 != 0 || chunk > cmax)
      return fail(FD_ERR_UNSUPPORTED, "FFD chunk=%d must be a multiple of 32 <= %d", chunk,
                  cmax);
  }
  if (int e = check_scale(scale)) return e;
  if (!(delta >= 0.f)) return fail(FD_ERR_ARG, "delta must be >= 0");
  if (n_sink < 0 || n_local < 0 || n_sink + n_local < 1)
    return fail(FD_ERR_ARG, "need n_sink, n_local >= 0 and n_sink + n_local >= 1");
  const int nc = n_chunks_of(L, chunk);
  if (int e = check_units(B, Hq, nc)) return e;
  const size_t need = partial_bytes(B, Hq, nc, d) + 2 * align256((size_t)B * Hq * 4);
  if (int e = workspace_gate(ws, ws_bytes, need)) return e;
  if (ws == nullptr) return ok();
  if (!q || !codes || !zs || !res || !rs || !v || !out)
    return fail(FD_ERR_ARG, "q, packed keys, v and out must not be NULL");
  if (!aligned16(q) || !aligned16(codes) || !aligned16(res) || !aligned16(v) ||
      !aligned16(out) || ((uintptr_t)zs & 3) != 0)
    return fail(FD_ERR_ARG, "q, codes, res, v, out must be 16-byte and zs 4-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float *o_part, *ml_part;
  split_ws(ws, B, Hq, nc, d, &o_part, &ml_part);
  char* tail = reinterpret_cast<char*>(ws) + partial_bytes(B, Hq, nc, d);
  fdk::FfdArgs fa{};
  fa.anchor_max = reinterpret_cast<float*>(tail);
  fa.anchor_pos = reinterpret_cast<int32_t*>(tail + align256((size_t)B * Hq * 4));
  fa.q = reinterpret_cast<const uint16_t*>(q);
  fa.codes = codes;
  fa.zs = zs;
  fa.res = res;
  fa.rs = rs;
  fa.v = reinterpret_cast<const uint16_t*>(v);
  fa.o_part = o_part;
  fa.ml_part = ml_part;
  fa.cand_mask = cand_mask;
  fa.pseudo_max = pseudo_max;
  fa.B = B;
  fa.Hq = Hq;
  fa.Hkv = Hkv;
  fa.L = L;
  fa.chunk = chunk;
  fa.nc = nc;
  fa.n_sink = n_sink;
  fa.n_local = n_local;
  fa.scale = scale;
  fa.c_log2 = (float)((double)scale * 1.4426950408889634);
  fa.delta_raw = isinf(delta) ? delta : (float)((double)delta / (double)scale);
  hipError_t e = fdk::launch_ffd(d, Hq / Hkv, fa, s);
  if (e != hipSuccess) return hip_status(e, "ffd kernel launch");
  fdk::MergeArgs ma{o_part, ml_part, out, lse, nullptr, Hq, nc, chunk, L, nullptr};
  return hip_status(fdk::launch_merge(d, B, ma, s), "merge kernel launch");
}

}  // extern "C"
