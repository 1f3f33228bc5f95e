/*
 * fd.h - C ABI of the MI355X (gfx950) single-query decode-attention library.
 *
 * One call computes, for every sequence b and query head h of a batch,
 *     out[b,h] = softmax(scale * q[b,h] . K_b^T) V_b,    lse[b,h] = ln sum exp(...)
 * over that sequence's cached keys and values, the way split-KV Flash-Decoding
 * does it: the cache is cut into chunks along the sequence, every chunk yields
 * a partial (m_i, l_i, O_i) in parallel, and the partials are merged exactly
 * through the exp(m_i - m) rescale.
 *   - Standard attention and its four steps: "Flash Decoding" explainer
 *     (aiqz.cc), section 1.
 *   - Split-KV partials and the exact merge: same page, section 2 (the
 *     displayed merge assumes normalised partials; this library keeps
 *     unnormalised O_i and divides by sum exp(m_i - m) l_i, which is the same
 *     value).
 *
 * Conventions shared by every entry point
 *   - All pointers except `ws_bytes` and `stream` are DEVICE pointers.  The
 *     caller allocates every buffer (fd_decode_attn_noalloc aside, whose
 *     partials buffer is a static array of the library); the library never
 *     allocates or frees.
 *   - Layouts are dense row-major with the shapes given below; element types
 *     are bf16 (raw 16-bit storage), fp32, fp16 (raw 16-bit storage), int8,
 *     int32 or uint32 as stated.  Alignment: q, k, v, pools, out and packed
 *     arrays 16 bytes; ws 256 bytes.
 *   - Grouped-query heads: query head h reads kv-head h / (Hq / Hkv).
 *   - `scale` is the score scale, normally 1/sqrt(d).  Scores, `phi`,
 *     margins and `delta` are all in units of scale * (q . k).
 *   - `out` is always fp32 [B, Hq, d]; `lse` (nullable) is fp32 [B, Hq].
 *   - Workspace, two phases: with ws == NULL the call stores the bytes it
 *     needs in *ws_bytes and returns FD_OK without touching the GPU; with
 *     ws != NULL it returns FD_ERR_WORKSPACE if *ws_bytes is smaller.  The
 *     workspace holds the per-chunk partials between the kernels of one call;
 *     its contents are not meaningful to the caller.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     returns without waiting.  Inputs must stay alive and unmodified until
 *     the stream has passed the call.  Calls on one stream may reuse one
 *     workspace; concurrent calls on different streams need their own.
 *   - Arguments are validated before anything is enqueued; a non-zero return
 *     means nothing was launched (except FD_ERR_HIP, reported after a launch
 *     failed).  fd_last_error() then describes the failure.
 *   - Non-finite values in q/K/V propagate; the kernels do not check data.
 *   - Supported: d in {64, 128}; group size G = Hq / Hkv in {1, 2, 4, 8}
 *     for every entry point, and for the dense ones (fd_decode_attn,
 *     fd_decode_attn_noalloc, fd_decode_attn_partials, fd_decode_attn_multi)
 *     also any other G with G * (query tokens) <= 32 on bf16 inputs, which
 *     runs on the matrix-core kernel (e.g. 28 query heads over 4 kv-heads,
 *     or 16 or 32 heads per kv-head); chunk a positive multiple of 16 no
 *     larger than 65536; B * (query rows per sequence) *
 *     (number of chunks) at most 2^31 - 1 (the kernels index partial rows
 *     with 32-bit integers), else FD_ERR_UNSUPPORTED.
 */
#ifndef FD_H_
#define FD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FD_F32 = 0, FD_BF16 = 1 } fd_dtype_t;

enum {
  FD_OK = 0,
  FD_ERR_ARG = 1,          /* null pointer, non-positive size, bad shape */
  FD_ERR_UNSUPPORTED = 2,  /* valid but not implemented (d, group size, dtype) */
  FD_ERR_WORKSPACE = 3,    /* *ws_bytes smaller than required */
  FD_ERR_HIP = 4           /* a HIP call or kernel launch failed */
};

/* Message for the last non-FD_OK return on the calling thread ("" if none).
 * The pointer stays valid until the next library call on that thread. */
const char* fd_last_error(void);

/* Library ABI version (increments on any signature or layout change). */
int fd_abi_version(void);

/*
 * Dense decode attention over a contiguous cache.
 *   dt      element type of q, k and v (FD_F32 or FD_BF16)
 *   q       [B, Hq, d]
 *   k, v    [B, Hkv, L, d]
 *   out     fp32 [B, Hq, d];   lse  fp32 [B, Hq] or NULL
 *   L       cached positions per sequence (>= 1)
 *   chunk   positions per split-KV chunk; chunk c covers
 *           [c*chunk, min((c+1)*chunk, L)), n_chunks = ceil(L / chunk).
 * The result does not depend on `chunk` beyond fp32 rounding.  A call with
 * fewer than 1,024 (sequence, kv-head, chunk) units (MI355X's SIMD count)
 * splits its chunks further, halving down to 32 positions while the halves
 * stay multiples of 16, so that every SIMD reads a share of the cache; the
 * workspace query accounts for it (the same rule holds for the paged entry
 * points, whose splits stay multiples of the page, with max_seq_len as L).
 * G in {1, 2, 4, 8}: the vector kernel, bf16 or fp32, except bf16 with
 * G = 8 on calls of at least 1,024 units, which take the matrix-core kernel
 * (eight heads per kv-head keep the vector kernel issue-bound).  Other
 * G <= 32 (bf16 only, else FD_ERR_UNSUPPORTED): the matrix-core kernel of
 * fd_decode_attn_multi with one token, whose splits may then cover several
 * consecutive chunks (same result up to fp32 rounding).  The same choice
 * holds for fd_decode_attn_noalloc and fd_decode_attn_partials (whose
 * partials stay per chunk).
 */
int fd_decode_attn(fd_dtype_t dt, const void* q, const void* k, const void* v,
                   float* out, float* lse,
                   int B, int Hq, int Hkv, int L, int d, float scale, int chunk,
                   void* ws, size_t* ws_bytes, void* stream);

/*
 * fd_decode_attn without a workspace and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments (minus ws,
 * ws_bytes), kernels and result as fd_decode_attn.  The chunk partials go to
 * a buffer the library owns: FD_NOALLOC_BYTES on every device the library
 * runs on, held until the process ends.  The call uses the current device's
 * buffer (`stream` must belong to the current device).
 *   - FD_ERR_WORKSPACE, with nothing launched, when the partials need more:
 *     round_up(B*Hq*n*d*4, 256) + round_up(B*Hq*n*8, 256) bytes, n the
 *     call's splits per sequence (fd_decode_attn's workspace size; 8.5 MB
 *     at B 8, Hq 32, d 128, 64 chunks).
 *   - Every call on one device shares that device's buffer, and it keeps the
 *     last call's contents (nothing in it needs clearing: every partial a
 *     call reads, that call writes first).  Calls that may overlap on one
 *     device (different streams, or several host threads) race and must be
 *     ordered by the caller.
 */
#define FD_NOALLOC_BYTES (32u << 20)

int fd_decode_attn_noalloc(fd_dtype_t dt, const void* q, const void* k, const void* v,
                           float* out, float* lse,
                           int B, int Hq, int Hkv, int L, int d, float scale, int chunk,
                           void* stream);

/*
 * The two stages of fd_decode_attn, for callers that merge partials
 * themselves -- e.g. partials of one sequence computed on several devices and
 * gathered along the chunk axis ("Flash Decoding" explainer, section 2: the
 * merge needs only (m_i, l_i, O_i) of every block).
 *
 * fd_decode_attn_partials takes the arguments of fd_decode_attn minus out
 * and lse, and leaves the chunk partials in ws (same workspace size):
 *   O   fp32 [B, Hq, n_chunks, d] at byte offset 0, O_c = sum_j 2^(s_j - m_c) v_j
 *   ML  fp32 [B, Hq, n_chunks, 2] at byte offset round_up(B*Hq*n_chunks*d*4, 256):
 *       (m_c, l_c) with m_c = log2(e) * max_j scale*q.k_j and
 *       l_c = sum_j 2^(s_j - m_c), where s_j = log2(e) * scale * q.k_j.
 * fd_merge_partials merges such partials into out fp32 [B, Hq, d] and lse
 * fp32 [B, Hq] (nullable):
 *   M = max_c m_c, out = sum_c 2^(m_c-M) O_c / sum_c 2^(m_c-M) l_c,
 *   lse = ln 2 * (M + log2 sum_c 2^(m_c-M) l_c).
 * A row whose chunks are all empty (every l_c = 0, m_c = -inf) gets out = 0
 * and lse = -inf.  n_chunks >= 1; o_part and ml_part 16-byte aligned.
 */
int fd_decode_attn_partials(fd_dtype_t dt, const void* q, const void* k,
                            const void* v, int B, int Hq, int Hkv, int L, int d,
                            float scale, int chunk, void* ws, size_t* ws_bytes,
                            void* stream);

int fd_merge_partials(const float* o_part, const float* ml_part, float* out,
                      float* lse, int B, int Hq, int n_chunks, int d, void* stream);

/*
 * Dense decode attention over a paged cache ("Flash Decoding" explainer,
 * section 3: the cache is cut into fixed-size pages allocated on demand).
 *   dt              FD_BF16 or FD_F32 (element type of q and both pools)
 *   k_pool, v_pool  [num_pages, Hkv, page_size, d]: one page holds page_size
 *                   consecutive positions of every kv-head of one sequence
 *   block_table     int32 [B, max_pages_per_seq]: position t of sequence b
 *                   is slot t % page_size of page block_table[b, t / page_size]
 *   seq_lens        int32 [B], device; 0 is allowed (out = 0, lse = -inf)
 *   max_seq_len     host-side upper bound of seq_lens (sizes grid and
 *                   workspace); must not exceed max_pages_per_seq * page_size
 *   page_size       a power of two in [8, 1024]; chunk % page_size == 0
 * bf16 with G = 8, at least 1,024 (sequence, kv-head, chunk) units over
 * max_seq_len, pages of 16 or more and chunk / page_size <= 256 runs as
 * fd_decode_attn_multi_paged with one token (its kernel, workspace and
 * result); otherwise the vector kernel.
 * Device-side values are clamped so that nothing is read out of bounds: a
 * length above max_seq_len is treated as max_seq_len and a page id outside
 * [0, num_pages) as the nearest valid id (the result is then meaningless).
 */
int fd_decode_attn_paged(fd_dtype_t dt, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_table,
                         const int32_t* seq_lens, float* out, float* lse,
                         int B, int Hq, int Hkv, int d, int page_size,
                         int max_pages_per_seq, int num_pages, int max_seq_len,
                         float scale, int chunk,
                         void* ws, size_t* ws_bytes, void* stream);

/*
 * Decode attention with a fixed ("unified") maximum and overflow fallback
 * ("FlashDecoding" deployment blog, section 1 and the fixed_max_value /
 * fallback_on_overflow settings of section 3): every chunk takes its
 * exponentials against the caller's constant phi instead of its own maximum,
 * so chunks need no shared running maximum and the merge needs no rescale.
 * A chunk is out of range for head h when its largest score exceeds
 * phi + margin_hi or falls below phi - margin_lo; such chunks are recomputed
 * exactly with their own maximum, inside the same kernel, before the merge.
 * The result is the dense result (softmax is shift invariant) for any finite
 * phi.  bf16 with G = 8 on a call of at least 1,024 units (where the vector
 * kernel is issue-bound) computes every chunk with its own maximum on the
 * matrix-core kernel instead, and sets the flags from the chunks' maxima
 * by the same range test.
 *   Arguments as fd_decode_attn, plus
 *   phi, margin_hi, margin_lo   finite; margins >= 0
 *   chunk_flags   uint8 [B, Hq, n_chunks] or NULL: 1 where the chunk was out
 *                 of range for that head, else 0.
 */
int fd_decode_attn_unified_max(fd_dtype_t dt, const void* q, const void* k,
                               const void* v, float* out, float* lse,
                               int B, int Hq, int Hkv, int L, int d, float scale,
                               int chunk, float phi, float margin_hi,
                               float margin_lo, uint8_t* chunk_flags,
                               void* ws, size_t* ws_bytes, void* stream);

/*
 * Multi-row decode attention: M new query tokens per sequence whose keys and
 * values are already in the cache at positions L-M .. L-1; token r attends to
 * positions 0 .. L-M+r ("Flash Decoding" explainer, section 1: a query sees
 * every key up to its own position).  The G*M query rows of a kv-head share
 * each K and V row (the flat-GEMM case of the "FlashDecoding" deployment
 * blog, section 1), computed on the matrix cores; M = 1 with G in
 * {1, 2, 4, 8} takes the single-query vector kernel of fd_decode_attn.
 *   q     [B, M, Hq, d]; k, v [B, Hkv, L, d]; L >= M
 *   out   fp32 [B, M, Hq, d];  lse fp32 [B, M, Hq] or NULL
 *   M = 1 and G in {1, 2, 4, 8}: dt bf16 or fp32 (the kernel fd_decode_attn
 *   picks).  Otherwise bf16 only and
 *   G*M <= 32, else FD_ERR_UNSUPPORTED.  Workspace: chunk partials of the B*M*Hq rows
 *   (same layout as fd_decode_attn_partials with M*Hq heads), sized for
 *   `chunk`.  On the matrix cores chunk is the split granule: when the rows' chunks
 *   outnumber what the device runs at once, one split covers F consecutive
 *   chunks, F chosen for the fewest rounds of splits (the latency estimate
 *   of the "Flash Decoding" explainer, section 2: splits beyond the
 *   hardware's parallelism only add merge work).  The result is the same up
 *   to fp32 rounding.
 *   chunk: each chunk writes G*M partial rows of (d + 2) floats per kv-head
 *   and the merge reads them back, so large M favours long chunks (on
 *   MI355X at L = 32768, B = 8: 2048 beat 512 by 4 % at M = 2 and 12 % at
 *   M = 8).
 */
int fd_decode_attn_multi(fd_dtype_t dt, const void* q, const void* k,
                         const void* v, float* out, float* lse, int B, int M,
                         int Hq, int Hkv, int L, int d, float scale, int chunk,
                         void* ws, size_t* ws_bytes, void* stream);

/*
 * fd_decode_attn_multi over a paged cache (the pools, block table and
 * lengths of fd_decode_attn_paged): sequence b holds seq_lens[b] positions,
 * its M new tokens' keys and values among them at seq_lens[b]-M ..
 * seq_lens[b]-1, and token r attends to positions 0 .. seq_lens[b]-M+r
 * ("Flash Decoding" explainer, sections 1 and 3).  A token with no position
 * to attend to (seq_lens[b]-M+r < 0) gets out = 0, lse = -inf.
 *   q    [B, M, Hq, d];  out fp32 [B, M, Hq, d];  lse fp32 [B, M, Hq] or NULL
 *   M = 1 and G in {1, 2, 4, 8}: the vector kernel of fd_decode_attn_paged
 *   (bf16 or fp32, page_size in [8, 1024]; bf16 with G = 8 takes the
 *   matrix-core kernel where fd_decode_attn_paged does).  Otherwise the
 *   matrix-core kernels:
 *   bf16, G*M <= 32, page_size a power of two in [16, 1024] and chunk /
 *   page_size <= 256, else FD_ERR_UNSUPPORTED.  The chunk is the split (the
 *   lengths live on the device): the pages that hold positions are
 *   divided evenly over the device's workers, so a worker may take a split
 *   from a page inside it on, and a second kernel folds that part into the
 *   split's partials with the same exact merge; the kernels also lengthen
 *   the split to chunk * F (F a power of two up to 256; at most 256 pages
 *   per split on the one-tile kernel, 512 on the wave pair) as long as
 *   every worker still gets a split's pages.
 * Workspace: the partials of B*M*Hq rows over nc = ceil(max_seq_len / chunk)
 * chunks (layout of fd_decode_attn_partials with M*Hq heads; a longer split
 * uses the first slots of each row); on the matrix-core kernels followed by
 * S = min(B*Hkv*nc (at least 1), 2048) worker slots: 256-byte-aligned blocks
 * of S*R*d and S*R*2 floats and S*4 int32 (R = G*M), and 256 bytes.
 * Device-side values are clamped as in fd_decode_attn_paged.
 */
int fd_decode_attn_multi_paged(fd_dtype_t dt, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, float* out, float* lse,
                               int B, int M, int Hq, int Hkv, int d, int page_size,
                               int max_pages_per_seq, int num_pages, int max_seq_len,
                               float scale, int chunk, void* ws, size_t* ws_bytes,
                               void* stream);

/*
 * Cache append ("Flash Decoding" explainer, section 3: each generated token
 * adds its key and value rows to the cache; a paged cache keeps them in
 * fixed-size pages listed by the block table).  Writes the step's M new rows
 * per (sequence, kv-head); the FFD key format of appended keys is made with
 * fd_ffd_pack over the same position range.
 *
 * fd_kv_append: contiguous cache, every sequence at the same position.
 *   k_new, v_new       [B, Hkv, M, d] (dt)
 *   k_cache, v_cache   [B, Hkv, L_cap, d] (dt); rows t .. t+M-1 are written
 *   0 <= t and t + M <= L_cap, else FD_ERR_ARG (nothing written)
 * fd_kv_append_paged: pools [num_pages, Hkv, page_size, d]; sequence b
 *   writes positions pos[b] .. pos[b]+M-1 (pos: int32 [B], device) to slot
 *   p % page_size of page block_table[b, p / page_size].  A position below
 *   0, past the table row (p / page_size >= max_pages_per_seq) or whose
 *   table entry is not in [0, num_pages) is skipped, not written.
 * All arrays 16-byte aligned; caller-owned; asynchronous on `stream`.  The
 * new rows must not overlap the cache rows they are written to.
 */
int fd_kv_append(fd_dtype_t dt, const void* k_new, const void* v_new,
                 void* k_cache, void* v_cache, int B, int Hkv, int M,
                 int L_cap, int d, int t, void* stream);

int fd_kv_append_paged(fd_dtype_t dt, const void* k_new, const void* v_new,
                       void* k_pool, void* v_pool, const int32_t* block_table,
                       const int32_t* pos, int B, int Hkv, int M, int d,
                       int page_size, int max_pages_per_seq, int num_pages,
                       void* stream);

/*
 * FFD key format ("Faster Than Flash" digest, section 5 and Fig. 2: a 2-bit
 * main part scanned for every position plus an 8-bit residual read only for
 * candidates).  Per position, per group of 32 consecutive dimensions:
 *   zero z = fp16(min x), step s = fp16((max x - min x) / 3)
 *   code c = clamp(rne((x - z) / s), 0, 3)       (c = 0 when s == 0)
 *   r = x - fma(s, c, z);  rs = fp16(max |r| / 127)
 *   r8 = clamp(rne(r / rs), -127, 127)           (r8 = 0 when rs == 0)
 * every step in fp32, round to nearest even.  2-bit key = z + s*c, refined
 * key = z + s*c + rs*r8.  Arrays, all [B, Hkv, L_cap, ...]:
 *   codes uint32 [.., d/16]: word w holds dims 16w..16w+15; dim 16w+2p at
 *         bits 2p..2p+1, dim 16w+2p+1 at bits 16+2p..17+2p (p = 0..7)
 *   zs    fp16   [.., d/32, 2]   (z, s)
 *   res   int8   [.., d]
 *   rs    fp16   [.., d/32]
 *
 * fd_ffd_pack quantises bf16 keys k [B, Hkv, L_cap, d] at positions
 * [t_begin, t_end) of every (b, kv-head) into those arrays (a whole cache, or
 * the positions appended this step).  Keys must be finite with |x| < 65504.
 * d in {64, 128}; 0 <= t_begin <= t_end <= L_cap.  No workspace.
 */
int fd_ffd_pack(const void* k, uint32_t* codes, uint16_t* zs, int8_t* res,
                uint16_t* rs, int B, int Hkv, int L_cap, int d, int t_begin,
                int t_end, void* stream);

/*
 * FFD sparse decode ("Faster Than Flash" digest, sections 3-6, Fig. 2), per
 * query head h of sequence b, over positions [0, L):
 *   1. pseudo-max m^ = max of the refined scores at the anchors: the first
 *      n_sink positions and the last n_local positions (section 4);
 *      j* = the lowest anchor position attaining it
 *   2. 2-bit scan score s~_j for every position (section 5)
 *   3. candidates C = { j : s~_j >= m^ - delta } plus j* (section 3)
 *   4. refined scores s^_j (2-bit + 8-bit residual key) for j in C
 *   5. exact softmax over C with the refined scores, merged over chunks
 *      with the exact rescale; out/lse as for the dense call.
 *   q          bf16 [B, Hq, d];  v  bf16 [B, Hkv, L, d]
 *   packed key arrays as for fd_ffd_pack, with L_cap = L
 *   delta      >= 0 (the pages use 5 and 7);  n_sink, n_local >= 0,
 *              n_sink + n_local >= 1
 *   cand_mask  uint32 [B, Hq, ceil(L/32)] or NULL: bit j%32 of word j/32 set
 *              when position j is in C
 *   pseudo_max fp32 [B, Hq] or NULL: m^
 *   chunk      positions per chunk: a multiple of 32, at most 2048
 *              (1024 when Hq / Hkv = 8); FD_ERR_UNSUPPORTED otherwise
 */
int fd_ffd_sparse_decode(const void* q, const uint32_t* codes,
                         const uint16_t* zs, const int8_t* res,
                         const uint16_t* rs, const void* v, float* out,
                         float* lse, int B, int Hq, int Hkv, int L, int d,
                         float scale, float delta, int n_sink, int n_local,
                         int chunk, uint32_t* cand_mask, float* pseudo_max,
                         void* ws, size_t* ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FD_H_ */
