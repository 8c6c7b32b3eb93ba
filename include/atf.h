/*
 * atf.h -- C ABI of librfw_atf.so: causal attention with per-RoPE-wavelength
 * distance windows (the ATFlash idea) for AMD Instinct MI355X (gfx950).
 *
 * The operation.  Source page: "ATFlash: RoPE-Frequenzen kuerzen
 * Attention-Arbeit um bis zu 57 Prozent" (sudo-ai.de).
 *   Section "Was ATFlash anders macht": RoPE rotates each pair of head dims at
 *   its own frequency; each pair gets a distance window derived from its
 *   wavelength, beyond which that pair's share of the query-key product is
 *   left out; slow pairs keep distant keys reachable (unlike a sliding window).
 *   Section "Die Zahlen - und ihre Grenze": prefill and decode attention keep
 *   their online-softmax recurrence unchanged.
 *   Readings used where the page gives no formula:
 *     P = d/2 pairs; pair p = head dims (p, p + P) in the half-split (NeoX)
 *     layout, or (2p, 2p + 1) in the interleaved (GPT-J) layout -- the
 *     formulas below write the half-split dims; the interleaved layout uses
 *     the same theta_p, W_p and rotation on its own pair of dims,
 *     theta_p = rope_base^(-2p/d), lambda_p = 2*pi/theta_p,
 *     W_p = ceil(alpha * lambda_p) for p < P-1, W_{P-1} = infinity,
 *     rotation by +angle (pos * theta_p):
 *       x'_p = x_p cos - x_{p+P} sin,  x'_{p+P} = x_{p+P} cos + x_p sin,
 *     score(i,j) = sum over p with (pos_i - pos_j) <= W_p of
 *                  q'_p k'_p + q'_{p+P} k'_{p+P},
 *     out_i = softmax_j(score(i,j) / sqrt(d)) . v_j over keys j with pos_j <= pos_i.
 *
 * Conventions shared by every call.
 *   - Tensors are DEVICE pointers owned by the caller, densely packed, 16-byte
 *     aligned:  q, out [B][Hq][Sq][d];  k, v [B][Hkv][S][d].
 *     q and k are given BEFORE the rotary embedding; the library rotates them.
 *   - GQA: query head h reads key/value head h / (Hq / Hkv).
 *   - dtype is the element type of q, k, v and out (fp32 accumulation always).
 *   - Positions: key j sits at pos0 + j.  Prefill query i sits at pos0 + i;
 *     the decode query sits at pos0 + S (right after the S cached keys).
 *   - All work is queued on `stream` (hipStream_t; NULL = default stream) and
 *     is asynchronous, except that a non-NULL skipped_out makes the call wait
 *     for the stream and copy the count back.
 *   - The library never allocates device memory inside a call: scratch space
 *     is the caller's `workspace` (size from the *_workspace_bytes query).
 *   - Errors are status codes only; nothing throws or aborts.  Every argument
 *     check runs on the host before anything is queued.
 *   - Supported: d in {64, 128, 256}; Hq % Hkv == 0; Hq/Hkv <= 64; S >= 1;
 *     0 <= pos0 and pos0 + S + 1 < 2^31; alpha > 0 (finite or +inf; +inf
 *     means no window); rope_base > 1 and finite; causal in {0, 1}.
 *   - rope_layout (calls that read q or k rows): ATF_ROPE_NEOX or
 *     ATF_ROPE_GPTJ, the same for q and k (see atf_rope_layout).
 *   - causal = 1: query i sees the keys at or before its position.  causal = 0
 *     (prefill): every key, the windows applying to the distance |i - j| (no
 *     page fixes the non-causal case; it is the plain reading of a distance
 *     window).  Decode is the same either way: its query follows every key.
 */
#ifndef ATF_H
#define ATF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *atf_stream_t; /* same object as hipStream_t */

typedef enum {
    ATF_OK = 0,
    ATF_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or value */
    ATF_ERR_UNSUPPORTED = 2, /* valid but not implemented (d, dtype, ...) */
    ATF_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    ATF_ERR_HIP = 4          /* a HIP launch or copy failed */
} atf_status;

typedef enum { ATF_F32 = 0, ATF_BF16 = 1 } atf_dtype;

/* How a head's d dims form the rotary pairs (argument `rope_layout`, int32_t).
 * The pages treat a pair as the unit a window cuts without fixing where its
 * two dims are stored; both common layouts are accepted.  Any other value is
 * ATF_ERR_INVALID_ARG.  In the interleaved layout a key's kept pairs are one
 * contiguous suffix of its row. */
typedef enum {
    ATF_ROPE_NEOX = 0, /* pair p = dims (p, p + d/2)  (rotate-half) */
    ATF_ROPE_GPTJ = 1  /* pair p = dims (2p, 2p + 1)  (interleaved) */
} atf_rope_layout;

/* Human-readable name of a status code (static string, never NULL). */
const char *atf_status_string(atf_status s);

/* Library version string (static). */
const char *atf_version(void);

/*
 * Window table: W_out[p] for p < d/2, computed in fp64 on the host.
 * INT64_MAX marks an uncut pair (always the slowest pair, every pair when
 * alpha is +inf).  Any even d >= 2 is accepted here.
 */
atf_status atf_window_table(int32_t d, double rope_base, double alpha, int64_t *W_out);

/*
 * Closed-form number of dropped (query, key, pair) terms for ONE (batch,
 * query-head) pair:  causal prefill of S tokens (is_decode = 0):
 * sum_p n_p (n_p + 1) / 2 with n_p = max(0, S - 1 - W_p);  decode of one query
 * after S keys (is_decode = 1): sum_p max(0, S - W_p).  causal = 0 doubles
 * the prefill count (the keys after each query, at the same distances) and
 * leaves decode unchanged.
 */
atf_status atf_skipped_pair_products(int64_t S, int32_t d, double rope_base, double alpha,
                                     int32_t causal, int32_t is_decode, uint64_t *per_head_out);

/* ------------------------------------------------------------------ prefill */

/* Bytes of workspace atf_prefill needs (rotated keys, re-laid-out values,
 * counters).  Returns 0 for unsupported shapes. */
size_t atf_prefill_workspace_bytes(int32_t B, int32_t Hkv, int64_t S, int32_t d, atf_dtype dtype);

/*
 * Causal windowed-RoPE prefill attention over S tokens:  out = attention(q, k, v).
 * Equivalent to atf_prefill_prepare_kv followed by atf_prefill_attend.
 * skipped_out (HOST pointer, nullable): receives the number of dropped
 * (query, key, pair) terms summed over all B*Hq heads, as counted by the
 * kernels; setting it synchronises `stream`.
 */
atf_status atf_prefill(const void *q, const void *k, const void *v, void *out,
                       int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t d,
                       int32_t rope_layout, double rope_base, double alpha, int32_t causal, int64_t pos0,
                       atf_dtype dtype, void *workspace, size_t workspace_bytes,
                       uint64_t *skipped_out, atf_stream_t stream);

/*
 * First half of atf_prefill: rotates every key at pos0 + j once and stores it
 * in `workspace` in the layout the attention kernel reads (bf16: rotated keys
 * with each pair's two dims side by side, values transposed per 64-key tile),
 * and clears the skipped-term counter (fp32: only clears the counter; the
 * fp32 kernel rotates keys as it streams them).
 */
atf_status atf_prefill_prepare_kv(const void *k, const void *v,
                                  int32_t B, int32_t Hkv, int64_t S, int32_t d,
                                  int32_t rope_layout, double rope_base, int64_t pos0, atf_dtype dtype,
                                  void *workspace, size_t workspace_bytes, atf_stream_t stream);

/*
 * Second half of atf_prefill: the attention kernel itself, reading q plus the
 * workspace prepared by atf_prefill_prepare_kv with the same B, Hkv, S, d,
 * rope_base, pos0 and dtype.  k and v are the raw inputs: the fp32 kernel
 * reads (and rotates) them directly; the bf16 kernel ignores them (NULL ok).
 * One prepared workspace serves any number of calls (other q, alpha or
 * causal); skipped_out counts the terms of this call only.
 */
atf_status atf_prefill_attend(const void *q, const void *k, const void *v, void *out,
                              int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t d,
                              int32_t rope_layout, double rope_base, double alpha, int32_t causal, int64_t pos0,
                              atf_dtype dtype, void *workspace, size_t workspace_bytes,
                              uint64_t *skipped_out, atf_stream_t stream);

/*
 * Chunked prefill: Sq new query tokens after a prefix of Sk - Sq cached
 * tokens, attending to the Sk keys (prefix + chunk): causally (causal = 1)
 * or to all of them with windows on |i - j| (causal = 0).
 *   q, out [B][Hq][Sq][d];  k, v [B][Hkv][Sk][d] (pre-RoPE, prefix first).
 * Key j sits at pos0 + j; query i at pos0 + Sk - Sq + i, so query i sees keys
 * 0 .. Sk - Sq + i and the windows apply to that distance exactly as in
 * atf_prefill (Sq == Sk is atf_prefill).  Source page "ATFlash: ..."
 * (sudo-ai.de), section "Die Zahlen - und ihre Grenze": the method drops into
 * the prefill path unchanged, and a prefill continued over a cached prefix is
 * that path with a query offset.  Needs 1 <= Sq <= Sk and at least
 * atf_prefill_workspace_bytes(B, Hkv, Sk, d, dtype) bytes of workspace (the
 * rotated keys of all Sk tokens).  Given atf_prefill_chunk_workspace_bytes
 * bytes or more, the bf16 path splits each query tile's key range over
 * several workgroups when the chunk is too short to fill the GPU, and merges
 * the splits' partial results (unnormalised output, reference maximum, sum)
 * in a combine kernel; the result is the same softmax up to fp32 rounding
 * order.  Errors: Sq < 1 or Sq > Sk is ATF_ERR_INVALID_ARG; otherwise as
 * atf_prefill with S = Sk.
 */
/*
 * Workspace bytes with which atf_prefill_chunk may split the key range: the
 * prepared keys and values of atf_prefill_workspace_bytes(B, Hkv, Sk, d,
 * dtype), followed by B*Hq*Sq*n_split rows of d + 2 floats of partials when
 * the planner splits (n_split <= 64) and, for a split chunk on 16-query waves
 * (d = 256, or d = 128 with Sq <= 16), from the next 256-byte boundary
 * B*Hq*Sq*d/2 words of queries rotated once for all splits.  Equal to atf_prefill_workspace_bytes
 * when no split would help (fp32, or a chunk that already fills the GPU).
 * Returns 0 for shapes atf_prefill_chunk rejects.
 */
size_t atf_prefill_chunk_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d,
                                         atf_dtype dtype);

atf_status atf_prefill_chunk(const void *q, const void *k, const void *v, void *out,
                             int32_t B, int32_t Hq, int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d,
                             int32_t rope_layout, double rope_base, double alpha, int32_t causal, int64_t pos0,
                             atf_dtype dtype, void *workspace, size_t workspace_bytes,
                             uint64_t *skipped_out, atf_stream_t stream);

/* --------------------------------------------- prefill over a kept key cache */

/*
 * A prefill key cache: the form atf_prefill_prepare_kv writes (keys rotated
 * once at their positions, pair-interleaved; values transposed per 64-key
 * tile), kept across calls so that a chunked prefill rotates only its own
 * new keys.  Same method as atf_prefill_chunk (source page "ATFlash: ..."
 * (sudo-ai.de), section "Die Zahlen - und ihre Grenze": the windows drop
 * into the prefill path unchanged, a chunk is that path with a query
 * offset); only where the keys come from differs.  bf16 only.
 *
 * Layout, for capacity S_cap keys per (b, kv head), S_pad = S_cap rounded up
 * to 128: rotated keys [B][Hkv][S_pad][d], then values [B][Hkv][S_pad / 64]
 * [d][64] (bf16).  Key j sits at position pos0 + j.  The caller owns the
 * cache; calls on one cache are ordered by their stream.
 */
size_t atf_prefill_cache_bytes(int32_t B, int32_t Hkv, int64_t S_cap, int32_t d);

/*
 * Writes keys k_begin .. k_begin + n - 1 of the cache from k, v
 * [B][Hkv][n][d] (pre-RoPE, bf16; row r is key k_begin + r at position
 * pos0 + k_begin + r).  Keys before k_begin are kept.  The cache then holds
 * k_begin + n keys: the keys after them up to the end of their 128-key tile
 * are cleared, so an append must not start inside a longer filled prefix it
 * means to keep.  rope_layout is that of k (and of the q later attending).
 * Errors: n < 1, k_begin < 0 or k_begin + n > S_cap is ATF_ERR_INVALID_ARG;
 * cache_bytes < atf_prefill_cache_bytes(...) is ATF_ERR_WORKSPACE; shape and
 * argument rules as atf_prefill_prepare_kv with S = S_cap.
 */
atf_status atf_prefill_cache_append(const void *k, const void *v, int32_t B, int32_t Hkv, int64_t n,
                                    int64_t k_begin, int64_t S_cap, int32_t d, int32_t rope_layout,
                                    double rope_base, int64_t pos0, void *cache, size_t cache_bytes,
                                    atf_stream_t stream);

/*
 * Scratch bytes for atf_prefill_chunk_cached: 256 (the dropped-term counter)
 * plus, when the planner splits the key range, B*Hq*Sq*n_split rows of d + 2
 * floats of partials (n_split <= 64) and the rotated queries laid out as in
 * atf_prefill_chunk_workspace_bytes.  0 for rejected shapes.
 */
size_t atf_prefill_cached_scratch_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d);

/*
 * Chunked prefill over the first Sk keys of a cache: q, out [B][Hq][Sq][d]
 * bf16 are the last Sq of those Sk tokens (query i at position
 * pos0 + Sk - Sq + i), as atf_prefill_chunk with the same k, v would see
 * them; the result equals atf_prefill_chunk's bit for bit when both run with
 * the same split (the same scratch or workspace size class).  Keys 0 .. Sk - 1
 * must have been appended.  `scratch` (device, >= 256 bytes, 16-byte
 * aligned) takes the counter; with atf_prefill_cached_scratch_bytes(...)
 * bytes or more it also takes the split partials (and rotated queries).  Calls that share a
 * scratch buffer must be ordered.  Errors: Sq < 1, Sq > Sk or Sk > S_cap is
 * ATF_ERR_INVALID_ARG; a short cache or scratch is ATF_ERR_WORKSPACE; other
 * rules as atf_prefill_chunk.
 */
atf_status atf_prefill_chunk_cached(const void *q, void *out, int32_t B, int32_t Hq, int32_t Hkv, int64_t Sq,
                                    int64_t Sk, int64_t S_cap, int32_t d, int32_t rope_layout, double rope_base,
                                    double alpha, int32_t causal, int64_t pos0, const void *cache,
                                    size_t cache_bytes, void *scratch, size_t scratch_bytes,
                                    uint64_t *skipped_out, atf_stream_t stream);

/* ------------------------------------------------------------------- decode */

/* Bytes of workspace atf_decode and atf_decode_kcache need: the counter, the
 * queries rotated once per call (B*Hq*d bf16), and the per-split partial
 * results. */
size_t atf_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t d);

/*
 * Windowed-RoPE decode: one new query per sequence, at position pos0 + S,
 * attending to the S cached keys at pos0 .. pos0 + S - 1.
 *   q, out [B][Hq][1][d];  k, v [B][Hkv][S][d] (the cache, pre-RoPE keys).
 * bf16 runs the split-KV kernel (each split reads only the key dims still
 * inside their window) followed by a combine kernel; fp32 runs a plain
 * per-query kernel.  skipped_out as for atf_prefill.
 */
atf_status atf_decode(const void *q, const void *k, const void *v, void *out,
                      int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t d,
                      int32_t rope_layout, double rope_base, double alpha, int32_t causal, int64_t pos0,
                      atf_dtype dtype, void *workspace, size_t workspace_bytes,
                      uint64_t *skipped_out, atf_stream_t stream);

/* --------------------------------------------- decode over a windowed key cache */

/*
 * A key cache laid out so that decode reads only the key dims the windows
 * keep.  Source page "ATFlash: ..." (sudo-ai.de), section "Was ATFlash anders
 * macht": beyond its window a pair's query-key term is dropped, so a key at
 * distance D contributes only pairs [p*(D), P) (p*(D) = #{p : W_p < D}).  In
 * the [S][d] layout both 128-byte halves of a d=128 key row always hold kept
 * pairs, and memory is read in whole lines; this layout makes the kept pairs
 * of a block of keys one contiguous byte range.
 *
 * Layout (bf16, device memory owned by the caller): for each (b, kv head), cap
 * keys (cap a multiple of 64) in 64-key blocks; block c holds P/4 planes of
 * 1024 bytes; plane pg holds, for each of the 64 keys, 16 bytes: pairs
 * 4pg .. 4pg+3 of the key ROTATED at its position, each as (x'_p, x'_{p+P}):
 *   byte ((b*Hkv + h) * (cap/64) + j/64) * (P/4 * 1024) + pg * 1024 + (j%64) * 16.
 */

/* Bytes of a key cache of capacity cap keys (0 if cap is not a positive
 * multiple of 64 below 2^31 or d is not 64, 128 or 256). */
size_t atf_decode_kcache_bytes(int32_t B, int32_t Hkv, int64_t cap, int32_t d);

/*
 * Writes keys into the cache: k [B][Hkv][n][d] (pre-RoPE, bf16) are cache keys
 * k_begin .. k_begin + n - 1, rotated at positions pos0 + k_begin + i (an
 * append when k_begin is the current length).  Requires 0 <= k_begin,
 * k_begin + n <= cap, cap % 64 == 0, 0 <= pos0, pos0 + cap + 1 < 2^31.
 * dtype must be ATF_BF16 (ATF_F32 returns ATF_ERR_UNSUPPORTED).  Asynchronous
 * on `stream`.
 */
atf_status atf_decode_pack_k(const void *k, void *kcache, int32_t B, int32_t Hkv, int64_t n,
                             int64_t k_begin, int64_t cap, int32_t d, int32_t rope_layout, double rope_base,
                             int64_t pos0, atf_dtype dtype, atf_stream_t stream);

/*
 * The cache write of one serving decode step over this layout (source page
 * "ATFlash: RoPE-Frequenzen kuerzen Attention-Arbeit um bis zu 57 Prozent",
 * section "Die Zahlen - und ihre Grenze": the method lives in the serving
 * decode kernel, so each step's new key enters the cache it reads): keys k and
 * values v, both [B][Hkv][n][d] (pre-RoPE keys, bf16), become cache entries
 * k_begin .. k_begin + n - 1 -- keys rotated into kcache as atf_decode_pack_k
 * writes them, values copied as rows of vcache [B][Hkv][cap][d] (the value
 * layout atf_decode_kcache reads) -- in one launch.  A step appends the
 * token the previous step produced (n = 1, k_begin = the current length) and
 * then decodes with atf_decode_kcache.  Same requirements and errors as
 * atf_decode_pack_k; v and vcache must both be NULL (keys only, the same as
 * atf_decode_pack_k) or both non-NULL and 16-byte aligned, else
 * ATF_ERR_INVALID_ARG.  Asynchronous on `stream`.
 */
atf_status atf_decode_append_kv(const void *k, const void *v, void *kcache, void *vcache, int32_t B, int32_t Hkv,
                                int64_t n, int64_t k_begin, int64_t cap, int32_t d, int32_t rope_layout,
                                double rope_base, int64_t pos0, atf_dtype dtype, atf_stream_t stream);

/*
 * atf_decode over that cache: query q [B][Hq][1][d] at position pos0 + S over
 * cache keys 0 .. S-1 (S <= cap) of kcache and value rows 0 .. S-1 of
 * v [B][Hkv][cap][d] (standard layout, row stride cap).  Same result,
 * windows, workspace (atf_decode_workspace_bytes(B, Hq, Hkv, S, d)) and
 * skipped count as atf_decode; bf16 only.  Errors: cap not a multiple of 64,
 * S > cap or pos0 + cap + 1 >= 2^31 is ATF_ERR_INVALID_ARG; otherwise as
 * atf_decode.
 */
atf_status atf_decode_kcache(const void *q, const void *kcache, const void *v, void *out,
                             int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int64_t cap, int32_t d,
                             int32_t rope_layout, double rope_base, double alpha, int32_t causal, int64_t pos0,
                             atf_dtype dtype, void *workspace, size_t workspace_bytes,
                             uint64_t *skipped_out, atf_stream_t stream);

/* ------------------------------------------------------- paged, ragged decode */

/*
 * The key-cache layout in pages, as a serving engine keeps it: a pool of pages
 * of 64 tokens; sequence b's 64-token block c lives in page
 * page_table[b * max_pages + c] (device int32 array [B][max_pages]), and
 * sequence b holds seq_lens[b] tokens (device int32 array [B]).  Same method
 * and source passages as atf_decode_kcache: the windows decide which key
 * planes a block needs, so distant blocks read fewer bytes.
 * Page p of the key pool (atf_paged_page_bytes bytes) holds, for each kv head
 * h, one 64-key block in the plane layout of atf_decode_kcache at byte
 * (p * Hkv + h) * (P/4 * 1024); page p of the value pool holds the 64 value
 * rows of each kv head at byte (p * Hkv + h) * (64 * d * 2) + (j % 64) * d * 2.
 * Both pools and both arrays are caller-owned device memory.  Page indices
 * outside [0, num_pages) are clamped into it (no out-of-pool access; the
 * result for such a table is unspecified).
 */

/* Bytes of one page of the key pool (equal to one page of the value pool);
 * 0 for unsupported Hkv or d. */
size_t atf_paged_page_bytes(int32_t Hkv, int32_t d);

/* Bytes of workspace atf_decode_paged needs (counter, rotated queries, and
 * per-split partials sized for the widest split count one sequence of max_len
 * tokens can take); 0 for unsupported shapes. */
size_t atf_decode_paged_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len, int32_t d);

/*
 * Writes tokens k_begin .. k_begin + n - 1 of every sequence into their
 * pages: k, v [B][Hkv][n][d] (pre-RoPE keys, bf16), keys rotated at
 * positions pos0 + k_begin + i.  Requires k_begin + n <= max_pages * 64;
 * pos0 + max_pages * 64 + 1 < 2^31.  bf16 only (ATF_F32 is
 * ATF_ERR_UNSUPPORTED).  Asynchronous on `stream`.
 */
atf_status atf_paged_write(const void *k, const void *v, void *kpool, void *vpool,
                           const int32_t *page_table, int32_t max_pages, int32_t num_pages,
                           int32_t B, int32_t Hkv, int64_t n, int64_t k_begin, int32_t d,
                           int32_t rope_layout, double rope_base, int64_t pos0, atf_dtype dtype, atf_stream_t stream);

/*
 * Ragged decode over the paged cache: sequence b's query q[b] ([B][Hq][1][d])
 * sits at position pos0 + seq_lens[b] and attends to its seq_lens[b] keys.
 * max_len (host) bounds every seq_lens[b] (values outside [1, max_len] are
 * clamped into it) and sizes the split plan and the workspace:
 * atf_decode_paged_workspace_bytes(B, Hq, Hkv, max_len, d).  Splits are
 * planned on the device: each sequence takes a share of ~512 workgroups in
 * proportion to its length, split into equal algorithmic bytes, so lengths
 * and pages can change between calls without host work.  skipped_out as for atf_decode
 * (summed over the ragged batch).  Errors: as atf_decode with S = max_len;
 * max_len > max_pages * 64 or a misaligned/NULL array is ATF_ERR_INVALID_ARG.
 */
atf_status atf_decode_paged(const void *q, const void *kpool, const void *vpool, void *out,
                            const int32_t *page_table, const int32_t *seq_lens, int32_t max_pages,
                            int32_t num_pages, int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len,
                            int32_t d, int32_t rope_layout, double rope_base, double alpha, int32_t causal, int64_t pos0,
                            atf_dtype dtype, void *workspace, size_t workspace_bytes,
                            uint64_t *skipped_out, atf_stream_t stream);

/* ------------------------------------------------ decode that allocates nothing */

/* Bytes of the library's own device scratch array (one per GPU, held from the
 * library's first use on that GPU until the process ends). */
#define ATF_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * atf_decode_paged for callers that cannot allocate or own a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics and results as atf_decode_paged
 * (bit-identical outputs, same kernels) without workspace/workspace_bytes:
 * the counter, rotated queries and split partials live in the library's
 * static device array of ATF_NOALLOC_SCRATCH_BYTES on the current GPU.  The
 * caller still owns q, out, the pools and the arrays.  Nothing is allocated
 * (no hipMalloc, hipFree or allocating library call).
 * Limit: shapes with atf_decode_paged_workspace_bytes(B, Hq, Hkv, max_len, d)
 * > ATF_NOALLOC_SCRATCH_BYTES are ATF_ERR_WORKSPACE, checked on the host
 * before any HIP call (e.g. Hq = 28, Hkv = 4, d = 128: B <= 17).
 * `stream` must belong to the current device (else ATF_ERR_INVALID_ARG).
 * Every call on one GPU shares that GPU's array and leaves it holding its
 * partials: calls that overlap on one GPU (different streams, or several host
 * threads) race and give wrong results; order them on one stream.
 */
atf_status atf_decode_paged_noalloc(const void *q, const void *kpool, const void *vpool, void *out,
                                    const int32_t *page_table, const int32_t *seq_lens, int32_t max_pages,
                                    int32_t num_pages, int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len,
                                    int32_t d, int32_t rope_layout, double rope_base, double alpha, int32_t causal,
                                    int64_t pos0, atf_dtype dtype, uint64_t *skipped_out, atf_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATF_H */
