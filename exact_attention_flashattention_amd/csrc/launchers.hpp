// Internal launch entry points, one per kernel family.  Shapes and pointers
// are validated by the C ABI layer before any of these is called; each
// returns the HIP status of its launch.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

hipError_t launch_prefill(const void* q, const void* k, const void* v, void* o, bool bf16, int batch, int hq,
                          int hkv, int n, int d, float scale, bool causal, hipStream_t stream);

// Packed variable-length batch: Q, O [total_q, hq, d], K, V [total_k, hkv, d];
// sequence b owns rows cu_q[b] .. cu_q[b+1]-1 and cu_k[b] .. cu_k[b+1]-1.
hipError_t launch_prefill_varlen(const void* q, const void* k, const void* v, void* o, const int* cu_q,
                                 const int* cu_k, int total_q, int total_k, int max_q, int max_k, bool bf16, int batch,
                                 int hq, int hkv, int d, float scale, bool causal, int window, const float* alibi,
                                 hipStream_t stream);

hipError_t launch_decode_splitk(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                                int max_kv_len, bool bf16, int batch, int hq, int hkv, int d, float scale,
                                int num_splits, int chunk, float* part_m, float* part_l, float* part_o,
                                hipStream_t stream);

// Paged caches [num_pages, hkv, 1 << page_shift, d]; row j of sequence b is
// row j % page of page block_table[b * max_pages + j / page].  window > 0 and
// alibi (per query head slopes, or null) are the masking variants.
hipError_t launch_decode_splitk_paged(const void* q, const void* k_pages, const void* v_pages,
                                      const int* block_table, int max_pages, int num_pages, int page_shift,
                                      const int* kv_lens, bool bf16, int batch, int hq, int hkv, int d, float scale,
                                      int num_splits, int chunk, int window, const float* alibi, float* part_m,
                                      float* part_l, float* part_o, hipStream_t stream);

// 4-bit (E2M1 codes + fp32 row scales) caches [B, hkv, max_kv_len, d/2] and
// [B, hkv, max_kv_len]; `rotated`: rows stored in the normalised Hadamard domain.
hipError_t launch_decode_splitk_q4(const void* q, const void* k_codes, const float* k_scales, const void* v_codes,
                                   const float* v_scales, const int* kv_lens, int max_kv_len, bool bf16, int batch,
                                   int hq, int hkv, int d, float scale, bool rotated, int num_splits, int chunk,
                                   float* part_m, float* part_l, float* part_o, hipStream_t stream);

// The same over paged pools: codes [num_pages, hkv, 1 << page_shift, d/2] and
// scales [num_pages, hkv, 1 << page_shift]; row j of sequence b is row j % page
// of page block_table[b * max_pages + j / page].
hipError_t launch_decode_splitk_q4_paged(const void* q, const void* k_codes, const float* k_scales,
                                         const void* v_codes, const float* v_scales, const int* block_table,
                                         int max_pages, int num_pages, int page_shift, const int* kv_lens, bool bf16,
                                         int batch, int hq, int hkv, int d, float scale, bool rotated, int num_splits,
                                         int chunk, float* part_m, float* part_l, float* part_o, hipStream_t stream);

// Rows [rows, d] of 16-bit values -> E2M1 codes [.., d/2] and fp32 scales, row i
// written to row out_rows[i] (or i) of the outputs when inside [0, out_capacity).
hipError_t launch_quantize_q4(const void* x, int rows, int d, bool bf16, bool rotated, float norm, const int* out_rows,
                              int out_capacity, void* codes, float* scales, hipStream_t stream);

hipError_t launch_merge(const float* part_m, const float* part_l, const float* part_o, int rows, int d,
                        int num_splits, bool bf16, void* out, hipStream_t stream);

// Measurement helpers (calibrate.hip): a bf16 MFMA loop and a streaming read.
hipError_t launch_calib_mfma(float* out, int blocks, int iters, hipStream_t stream);
hipError_t launch_calib_read(const void* buf, size_t bytes, void* scratch, int blocks, hipStream_t stream);

}  // namespace attn
