/*
 * attn.h -- C ABI of libattn.so: exact softmax attention on MI355X (gfx950).
 *
 * The library computes O = softmax(Q·Kᵀ·scale)·V exactly, tile by tile, with
 * the online-softmax recurrence: a running maximum m, running sum l and
 * unnormalised output o per query row, rescaled by exp(m − m_new) whenever a
 * new key tile raises the maximum, and O = o / l at the end.  The score matrix
 * never reaches device memory.  Definitions: the three-line math block and
 * "The online softmax" of "Attention from the kernel's side: FlashAttention,
 * online softmax and fused dequant"; "Concept" and "Maths" of "Attention
 * kernels".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a device pointer, owned and allocated by the
 *   caller; every tensor is dense and row-major with the head dimension
 *   innermost.  No call allocates or frees device memory, and none
 *   synchronises.  (attn_decode_noalloc keeps its partial states in a fixed
 *   array that the library holds on each GPU for the life of the process.)
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each
 *   call only enqueues kernels on it and returns.  ATTN_OK means the launches
 *   were accepted; faults during execution surface at the caller's next
 *   synchronisation.
 * - All argument checks happen on the host before anything is launched; a
 *   failed check launches nothing and returns its status.  There is no silent
 *   fallback to another algorithm.
 * - Element types: ATTN_BF16 or ATTN_F16 storage; products are accumulated in
 *   fp32 and the softmax state is kept in fp32.  Outputs are rounded to the
 *   output type with round-to-nearest-even.
 * - Supported head dimensions: d = 64 and d = 128.
 * - Grouped-query attention: query head h reads KV head h / (hq / hkv)
 *   ("GQA in the kernel", section 5 of "Attention Computation in Practice");
 *   hq must be a multiple of hkv.
 * - Every tensor pointer must be 16-byte aligned (the kernels use 128-bit
 *   loads and stores).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL_PTR = 1,    /* a required pointer is NULL */
  ATTN_ERR_BAD_SHAPE = 2,   /* a size is < 1, hq % hkv != 0, or scale is not finite */
  ATTN_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, or an unknown element type */
  ATTN_ERR_MISALIGNED = 4,  /* a tensor pointer is not 16-byte aligned */
  ATTN_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch */
  ATTN_ERR_TOO_LARGE = 6,   /* a size exceeds what the kernels index (see each call) */
  ATTN_ERR_SCRATCH = 7      /* attn_decode_noalloc: partials exceed the fixed scratch buffer */
} attn_status;

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char* attn_status_string(int status);

/*
 * attn_prefill_fwd -- prefill forward over a square problem.
 *
 * Computes, for every batch b, query head h and query row i,
 *   O[b,h,i,:] = sum_j softmax_j(scale · Q[b,h,i,:]·K[b,kh,j,:]) · V[b,kh,j,:],
 * kh = h / (hq / hkv), over keys j in [0, n) -- or j <= i when `causal` is
 * non-zero (key j visible to query i iff j <= i: "Masking variants" in
 * section 5 of "Attention Computation in Practice").  The recurrence runs over
 * key tiles held in LDS; tiles wholly above the diagonal are skipped, tiles
 * wholly below it need no mask (the block classification of the same
 * section).
 *
 *   q, o : [batch, hq,  n, d]  elements of `dtype`; o is written, q is read
 *   k, v : [batch, hkv, n, d]  elements of `dtype`, read only
 *   scale: the score scale, normally 1/sqrt(d); must be finite
 *   causal: 0 = every key visible, non-zero = causal mask j <= i
 *
 * Limits: batch, hq, hkv, n >= 1; batch·hq·n·d and batch·hkv·n·d below 2^40
 * elements, n below 2^31 / d (else ATTN_ERR_TOO_LARGE).  O must not alias Q,
 * K or V.
 */
attn_status attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, int dtype, int batch,
                             int hq, int hkv, int n, int d, float scale, int causal, void* stream);

/*
 * attn_prefill_varlen_fwd -- prefill / append over a packed batch of
 * sequences of different lengths (the append / mixed kernel "with cu_seqlens"
 * of "The four attention kernels you actually use", section 5 of "Attention
 * Computation in Practice": chunked prefill, verifying a few speculative
 * tokens).
 *
 * Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key
 * rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1; call their counts nq and nk.
 * Its queries are the LAST nq of its nk positions (bottom-right alignment),
 * so with `causal` non-zero query i (0-based within the sequence) sees keys
 * j <= i + nk - nq; without it every one of the nk keys.  nq = nk is the
 * square problem of attn_prefill_fwd.  A query row that sees no key (nk = 0,
 * or i + nk - nq < 0) is written as 0.
 *
 *   q, o : [total_q, hq,  d]  elements of `dtype`, token-major (packed)
 *   k, v : [total_k, hkv, d]  elements of `dtype`, read only
 *   cu_seqlens_q, cu_seqlens_k : [batch + 1] int32, DEVICE memory,
 *          non-decreasing.  Preconditions: cu[0] >= 0, cu[batch] <= total,
 *          each nq <= max_seqlen_q and nk <= max_seqlen_k.  The kernel clamps
 *          every sequence into those bounds, so no access leaves the tensors.
 *   total_q >= 1, total_k >= 0 : rows of the packed tensors
 *   max_seqlen_q >= 1, max_seqlen_k >= 0 : bounds on nq and nk (the grid is
 *          sized from max_seqlen_q)
 *   scale, causal : as for attn_prefill_fwd
 *   window : 0 = no window; W > 0 = sliding window: query i (position
 *          p = i + nk - nq) sees keys p - W < j <= p.  Needs `causal`
 *          (else ATTN_ERR_UNSUPPORTED); negative is ATTN_ERR_BAD_SHAPE.
 *   alibi_slopes : NULL = none; else [hq] fp32 in DEVICE memory: query head
 *          h adds -alibi_slopes[h]·(p - j) to its score of key j (natural-log
 *          units, after the scale).  Both masking variants are those of
 *          "Masking variants", section 5 of "Attention Computation in
 *          Practice".
 *
 * Limits: total·heads·d below 2^40 for each tensor; max_seqlen_k·hkv·d·2 below
 * 2^31 bytes (else ATTN_ERR_TOO_LARGE).  O must not alias Q, K or V.
 */
attn_status attn_prefill_varlen_fwd(const void* q, const void* k, const void* v, void* o, const int* cu_seqlens_q,
                                    const int* cu_seqlens_k, int total_q, int total_k, int max_seqlen_q,
                                    int max_seqlen_k, int dtype, int batch, int hq, int hkv, int d, float scale,
                                    int causal, int window, const float* alibi_slopes, void* stream);

/*
 * Split-K ("Flash-Decoding") single-query decode, in two calls: partial states
 * per key slice, then their merge.  Splitting the cache sequence across
 * workgroups is what lets one query fill the GPU ("Prefill and decode are
 * different problems" on the first page; "The four attention kernels you
 * actually use" in section 5 of "Attention Computation in Practice"; "Concept"
 * on "Attention kernels").
 *
 * Split s of sequence b covers cache rows [s·C, min((s+1)·C, kv_lens[b]))
 * where C = attn_decode_chunk_len(max_kv_len, num_splits).
 */

/* A split count that reads a bf16/fp16 cache of this shape fastest (host
 * heuristic, >= 1): about 512 waves, at most 4096 keys per split. */
int attn_decode_num_splits(int batch, int hkv, int max_kv_len);

/* The same for the 4-bit cache of attn_decode_splitk_q4, whose kernel needs
 * more waves in flight: about 2048 waves, at most 2048 keys per split. */
int attn_decode_q4_num_splits(int batch, int hkv, int max_kv_len);

/* Keys per split C for the given split count (a multiple of 64, >= 64);
 * returns 0 if max_kv_len < 1 or num_splits < 1. */
int attn_decode_chunk_len(int max_kv_len, int num_splits);

/* Bytes of partial state the caller must provide: part_m and part_l of
 * batch·hq·num_splits floats each, part_o of batch·hq·num_splits·d floats.
 * Returns 0 on a non-positive argument. */
size_t attn_decode_workspace_bytes(int batch, int hq, int d, int num_splits);

/*
 * attn_decode_splitk -- partial (m, l, o) of one query per (sequence, head)
 * over each split of its KV cache.
 *
 *   q       : [batch, hq, d]                elements of `dtype`
 *   k_cache : [batch, hkv, max_kv_len, d]   elements of `dtype`
 *   v_cache : [batch, hkv, max_kv_len, d]   elements of `dtype`
 *   kv_lens : [batch] int32, DEVICE memory; sequence b sees cache rows
 *             0 .. kv_lens[b]-1.  Precondition 0 <= kv_lens[b] <= max_kv_len;
 *             the kernel clamps each length into that range, and never reads
 *             a cache row at or past it.
 *   part_m, part_l : [batch, hq, num_splits] fp32, written
 *   part_o         : [batch, hq, num_splits, d] fp32, written
 *
 * Natural-log units: part_m is the largest scaled score (scale·q·k) in the
 * split, part_l = sum_j exp(s_j − m) and part_o = sum_j exp(s_j − m)·v_j
 * (unnormalised).  An empty split writes (m, l, o) = (−inf, 0, 0): the state
 * of a worker that saw no keys ("Maths" and "Code" on "Attention kernels").
 * Each workgroup reads the K/V tile of its KV head once and uses it for all
 * hq/hkv query heads that share it.
 *
 * Limits: batch, hq, hkv, max_kv_len, num_splits >= 1; batch·hkv·max_kv_len·d
 * below 2^40; max_kv_len below 2^31 / d (else ATTN_ERR_TOO_LARGE).
 */
attn_status attn_decode_splitk(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                               int max_kv_len, int dtype, int batch, int hq, int hkv, int d, float scale,
                               int num_splits, float* part_m, float* part_l, float* part_o, void* stream);

/*
 * attn_decode_splitk_paged -- attn_decode_splitk over a paged KV cache.
 *
 * The cache is a pool of fixed-size pages; each sequence lists its pages in a
 * block table, and the kernel gathers through it ("PagedAttention's kernel
 * difference" in section 5 of "Attention Computation in Practice").  Logical
 * cache row j of sequence b is row j % page_size of page
 * block_table[b·max_pages_per_seq + j / page_size].  Partials, splits and
 * units are exactly those of attn_decode_splitk with
 * max_kv_len = max_pages_per_seq · page_size, so the same merge applies and,
 * for the same logical cache contents and no masking variant, the partials
 * are bit-identical.  With a window, splits wholly before it are empty.
 *
 *   q           : [batch, hq, d]                        elements of `dtype`
 *   k_pages     : [num_pages, hkv, page_size, d]        elements of `dtype`
 *   v_pages     : [num_pages, hkv, page_size, d]        elements of `dtype`
 *   block_table : [batch, max_pages_per_seq] int32, DEVICE memory.  Only the
 *                 first ceil(kv_lens[b] / page_size) entries of row b are
 *                 used; each must lie in [0, num_pages) (out-of-range ids are
 *                 clamped into that range, so no read leaves the pool).
 *                 Pages may be shared between sequences.
 *   kv_lens     : [batch] int32, DEVICE memory; sequence b sees logical rows
 *                 0 .. kv_lens[b]-1, clamped into [0, max_pages_per_seq ·
 *                 page_size]; rows at or past it are never read.
 *   page_size   : a power of two >= 16 (else ATTN_ERR_UNSUPPORTED)
 *   window      : 0 = every key; W > 0 = sliding window: the query, at
 *                 position p = kv_lens[b] - 1, sees keys p - W < j <= p
 *                 (negative: ATTN_ERR_BAD_SHAPE)
 *   alibi_slopes: NULL = none; else [hq] fp32 in DEVICE memory: head h adds
 *                 -alibi_slopes[h]·(p - j) to its score of key j (natural-log
 *                 units, after the scale).  Both are the masking variants of
 *                 "Masking variants", section 5 of "Attention Computation in
 *                 Practice".
 *   part_m, part_l, part_o, num_splits : as for attn_decode_splitk
 *
 * Limits: max_pages_per_seq · page_size below 2^31 / d;
 * num_pages·hkv·page_size·d below 2^40 (else ATTN_ERR_TOO_LARGE).
 */
attn_status attn_decode_splitk_paged(const void* q, const void* k_pages, const void* v_pages,
                                     const int* block_table, int max_pages_per_seq, int num_pages, int page_size,
                                     const int* kv_lens, int dtype, int batch, int hq, int hkv, int d, float scale,
                                     int num_splits, int window, const float* alibi_slopes, float* part_m,
                                     float* part_l, float* part_o, void* stream);

/*
 * attn_decode_splitk_q4 -- attn_decode_splitk over a 4-bit KV cache,
 * dequantised inside the tile loads: the kernel reads only the codes and the
 * row scales ("Why a quantised cache needs a fused kernel" on "Attention from
 * the kernel's side": a separate dequantise pass would move more bytes than
 * the 16-bit cache it replaces).
 *
 *   q        : [batch, hq, d]                     elements of `dtype`
 *   k_codes  : [batch, hkv, max_kv_len, d/2] bytes; byte i of a row holds
 *              elements 2i (low nibble) and 2i+1 (high nibble), each an OCP
 *              MX E2M1 code (bit 3 sign, bits 2:1 exponent with bias 1, bit 0
 *              mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6)
 *   k_scales : [batch, hkv, max_kv_len] fp32; row value = code value × scale
 *   v_codes, v_scales : the same for V
 *   rotated  : 0 = rows hold k and v; 1 = rows hold R·k and R·v with
 *              R = H_d / sqrt(d), the normalised Sylvester-Hadamard matrix
 *              (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]).  The kernel
 *              rotates q by R on load and the partial outputs back by R (R is
 *              its own inverse), so q and the outputs are always unrotated.
 *   kv_lens, max_kv_len, num_splits, part_m, part_l, part_o : as for
 *              attn_decode_splitk; the partials are merged by
 *              attn_merge_partials.
 *
 * The result is attention over the dequantised cache (code value × scale,
 * rotated back when `rotated`), computed with the same split-K recurrence.
 * Every pointer must be 16-byte aligned.  Limits as for attn_decode_splitk.
 */
attn_status attn_decode_splitk_q4(const void* q, const void* k_codes, const float* k_scales, const void* v_codes,
                                  const float* v_scales, const int* kv_lens, int max_kv_len, int dtype, int batch,
                                  int hq, int hkv, int d, float scale, int rotated, int num_splits, float* part_m,
                                  float* part_l, float* part_o, void* stream);

/*
 * attn_decode_splitk_q4_paged -- attn_decode_splitk_q4 over a paged 4-bit
 * cache: the page pool and block table of attn_decode_splitk_paged ("PagedAttention's
 * kernel difference" in section 5 of "Attention Computation in Practice")
 * holding the codes and row scales of attn_decode_splitk_q4 ("Why a quantised
 * cache needs a fused kernel" on "Attention from the kernel's side").
 * Logical cache row j of sequence b is row j % page_size of page
 * block_table[b·max_pages_per_seq + j / page_size], in both the code pool and
 * the scale pool.  Partials, splits and units are those of
 * attn_decode_splitk_q4 with max_kv_len = max_pages_per_seq · page_size; for
 * the same logical cache contents the partials are bit-identical.
 *
 *   q           : [batch, hq, d]                          elements of `dtype`
 *   k_codes     : [num_pages, hkv, page_size, d/2] bytes (E2M1 pairs as for
 *                 attn_decode_splitk_q4)
 *   k_scales    : [num_pages, hkv, page_size] fp32
 *   v_codes, v_scales : the same for V
 *   block_table : [batch, max_pages_per_seq] int32, DEVICE memory; only the
 *                 first ceil(kv_lens[b] / page_size) entries of row b are
 *                 used; ids outside [0, num_pages) are clamped into it, so no
 *                 read leaves the pools.  Pages may be shared.
 *   kv_lens     : [batch] int32, DEVICE memory, clamped into
 *                 [0, max_pages_per_seq · page_size]
 *   page_size   : a power of two >= 16 (else ATTN_ERR_UNSUPPORTED)
 *   rotated, num_splits, part_m, part_l, part_o : as for
 *                 attn_decode_splitk_q4 (no masking variants)
 *
 * Every pointer must be 16-byte aligned.  Limits: max_pages_per_seq ·
 * page_size below 2^31 / d; num_pages·hkv·page_size·d below 2^40 (else
 * ATTN_ERR_TOO_LARGE).
 */
attn_status attn_decode_splitk_q4_paged(const void* q, const void* k_codes, const float* k_scales,
                                        const void* v_codes, const float* v_scales, const int* block_table,
                                        int max_pages_per_seq, int num_pages, int page_size, const int* kv_lens,
                                        int dtype, int batch, int hq, int hkv, int d, float scale, int rotated,
                                        int num_splits, float* part_m, float* part_l, float* part_o, void* stream);

/*
 * attn_kv_quantize_q4 -- encode rows of keys or values into the 4-bit cache
 * format read by attn_decode_splitk_q4 (the write side of the fused-dequant
 * cache: rows are quantised once, as they enter the cache).
 *
 *   x        : [rows, d] elements of `dtype`, DEVICE memory, read
 *   rotated  : 0 = encode x; 1 = encode R·x (R = H_d / sqrt(d) as above)
 *   out_rows : NULL (row i goes to output row i; then rows <= out_capacity)
 *              or [rows] int32 DEVICE memory: row i goes to output row
 *              out_rows[i]; a destination outside [0, out_capacity) is
 *              skipped (nothing written).  E.g. appending one position to a
 *              [batch, hkv, max_kv_len] cache: (b·hkv + kh)·max_kv_len + pos.
 *   codes    : [out_capacity, d/2] bytes, written (E2M1 pairs as above)
 *   scales   : [out_capacity] fp32, written
 *
 * Per row, in fp32 and in this order: with `rotated` the Walsh-Hadamard
 * butterflies over the element index bits from bit 0 upward (lower element
 * a, upper b -> a + b, a - b) and one multiplication by 1/sqrt(d) rounded to
 * fp32; scale = max|y| / 6 (1 for an all-zero row); each element's code is the
 * nearest E2M1 magnitude of |y / scale| (ties to the even code) with the sign
 * bit set when y / scale < 0.  Inputs must be finite.  x, codes and scales
 * must be 16-byte aligned.
 */
attn_status attn_kv_quantize_q4(const void* x, int rows, int d, int dtype, int rotated, const int* out_rows,
                                int out_capacity, void* codes, float* scales, void* stream);

/*
 * attn_decode_noalloc -- attn_decode_splitk followed by attn_merge_partials
 * in one call that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  The split-K partial states live in a
 * fixed scratch array inside the library (one per GPU, held until the
 * process ends) instead of caller memory; the caller passes only inputs and
 * the output.  No hipMalloc, hipFree or other allocating routine is called.
 *
 *   q, k_cache, v_cache, kv_lens, max_kv_len, dtype, batch, hq, hkv, d,
 *   scale : as for attn_decode_splitk
 *   num_splits : >= 1, or 0 for attn_decode_num_splits(batch, hkv, max_kv_len)
 *   o          : [batch, hq, d] elements of `dtype`, DEVICE memory, written
 *
 * The partials -- batch·hq·num_splits·(d + 2) fp32 values, each of the three
 * arrays 256-byte aligned -- must fit in ATTN_DECODE_NOALLOC_SCRATCH_BYTES
 * (64 MiB; e.g. batch 64, hq 64, 16 splits, d 128 takes 34 MB), else
 * ATTN_ERR_SCRATCH and nothing is launched.  Every call on one GPU uses the
 * same array: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and give undefined results.
 * Nothing in the array needs to start at zero -- every partial the merge
 * reads is written by the same call -- so a call never depends on what an
 * earlier one left there.  The first call on a device looks up the array's
 * address there (hipGetSymbolAddress); `stream` must belong to a device the
 * library runs on.  Results are bit-identical to attn_decode_splitk +
 * attn_merge_partials with the same num_splits.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)
attn_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                                int max_kv_len, int dtype, int batch, int hq, int hkv, int d, float scale,
                                int num_splits, void* o, void* stream);

/*
 * attn_merge_partials -- merge the partial states of each (sequence, head)
 * and normalise: m = max_s m_s, l = sum_s l_s·exp(m_s − m),
 * o = sum_s o_s·exp(m_s − m), O = o / l (the two-state merge rule of "Maths"
 * on "Attention kernels", applied across all splits).  A partial with
 * m_s = −inf contributes nothing; if every partial is empty (l = 0) the
 * output row is 0.
 *
 *   part_m, part_l : [batch, hq, num_splits] fp32, read
 *   part_o         : [batch, hq, num_splits, d] fp32, read
 *   o              : [batch, hq, d] elements of `out_dtype`, written
 */
attn_status attn_merge_partials(const float* part_m, const float* part_l, const float* part_o, int batch,
                                int hq, int d, int num_splits, void* o, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
