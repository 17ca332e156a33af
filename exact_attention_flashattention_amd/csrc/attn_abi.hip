// C ABI of libattn.so (declared in include/attn.h and include/attn_calibrate.h): argument validation on
// the host, split planning for decode, and dispatch to the kernel launchers.
// Nothing here allocates, frees or synchronises device memory.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn.h"
#include "attn_calibrate.h"
#include "launchers.hpp"

namespace {

constexpr long long kMaxElems = 1LL << 40;  // per-tensor element bound the kernels' 64-bit offsets assume
// Split plans.  bf16/fp16 caches: about 512 waves of up to 4096 keys each --
// two per CU, each streaming 1 MB of K and V at d = 128 -- read the cache
// faster than more, shorter splits (measured on one sequence of 262144 keys,
// 8 KV heads: 64 splits 5.9 TB/s by wall clock with the merge, 256 splits
// 5.7; on 64 ragged sequences of up to 32768 keys 8 and 16 splits tie).  The
// 4-bit cache's kernel does more arithmetic per byte and needs more waves in
// flight: about 2048 waves of up to 2048 keys (64 splits there: 2.9 TB/s of
// codes and scales, 256 splits: 4.4).
constexpr int kDecodeTargetWaves = 512;
constexpr int kDecodeMaxChunk = 4096;       // most keys per split, so ragged lengths balance across waves
constexpr int kDecodeQ4TargetWaves = 2048;
constexpr int kDecodeQ4MaxChunk = 2048;
constexpr int kDecodeMinChunk = 256;        // fewest keys worth a split of its own
constexpr int kChunkAlign = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int t) { return t == ATTN_F16 || t == ATTN_BF16; }
bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

// ---- fixed scratch of attn_decode_noalloc: the split-K partial states live in
// this array instead of caller memory.  Each GPU the library runs on holds its
// own copy for the life of the process.  Host code never passes the array's
// name to a kernel (on the host it names a stand-in, not device memory): the
// device address is taken once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device address of this library's scratch array on the device `stream`
// belongs to (the current device for the null stream).
attn_status scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_LAUNCH;
  int dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return ATTN_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return ATTN_ERR_LAUNCH;
    if (e != hipSuccess || p == nullptr) return ATTN_ERR_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case ATTN_ERR_BAD_SHAPE: return "bad shape or scale";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension or element type";
    case ATTN_ERR_MISALIGNED: return "tensor pointer not 16-byte aligned";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_TOO_LARGE: return "size beyond the kernels' index range";
    case ATTN_ERR_SCRATCH: return "partial states larger than the library's fixed scratch buffer";
    default: return "unknown status";
  }
}

attn_status attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, int dtype, int batch, int hq,
                             int hkv, int n, int d, float scale, int causal, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL_PTR;
  if (batch < 1 || hq < 1 || hkv < 1 || n < 1 || hq % hkv != 0 || !scale_ok(scale)) return ATTN_ERR_BAD_SHAPE;
  if ((d != 64 && d != 128) || !dtype_ok(dtype)) return ATTN_ERR_UNSUPPORTED;
  if ((long long)batch * hq * n * d >= kMaxElems || (long long)n * d >= (1LL << 31)) return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_MISALIGNED;
  return from_hip(attn::launch_prefill(q, k, v, o, dtype == ATTN_BF16, batch, hq, hkv, n, d, scale, causal != 0,
                                       static_cast<hipStream_t>(stream)));
}

attn_status attn_prefill_varlen_fwd(const void* q, const void* k, const void* v, void* o, const int* cu_seqlens_q,
                                    const int* cu_seqlens_k, int total_q, int total_k, int max_seqlen_q,
                                    int max_seqlen_k, int dtype, int batch, int hq, int hkv, int d, float scale,
                                    int causal, int window, const float* alibi_slopes, void* stream) {
  if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULL_PTR;
  if (batch < 1 || hq < 1 || hkv < 1 || total_q < 1 || total_k < 0 || max_seqlen_q < 1 || max_seqlen_k < 0 ||
      hq % hkv != 0 || !scale_ok(scale) || window < 0)
    return ATTN_ERR_BAD_SHAPE;
  if ((d != 64 && d != 128) || !dtype_ok(dtype) || (window > 0 && !causal)) return ATTN_ERR_UNSUPPORTED;
  // per-sequence K/V byte ranges are 32-bit buffer offsets; the grid is one-dimensional
  const long long tiles = (max_seqlen_q + 255) / 256 + 1;  // at least the kernel's query tiles (>= 256 rows each)
  const long long blocks = 8LL * (((long long)batch * hkv + 7) / 8) * (hq / hkv) * tiles;
  if ((long long)total_q * hq * d >= kMaxElems || (long long)total_k * hkv * d >= kMaxElems ||
      (long long)max_seqlen_k * hkv * d * 2 >= (1LL << 31) || blocks >= (1LL << 31))
    return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_MISALIGNED;
  return from_hip(attn::launch_prefill_varlen(q, k, v, o, cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q,
                                              max_seqlen_k, dtype == ATTN_BF16, batch, hq, hkv, d, scale,
                                              causal != 0, window, alibi_slopes, static_cast<hipStream_t>(stream)));
}

namespace {
int split_plan(int batch, int hkv, int max_kv_len, int target_waves, int max_chunk) {
  if (batch < 1 || hkv < 1 || max_kv_len < 1) return 1;
  // enough splits to fill the GPU, and enough that no split holds more than
  // the maximum chunk; never so many that splits drop below the minimum chunk
  const long long heads = (long long)batch * hkv;
  const long long fill = (target_waves + heads - 1) / heads;
  const long long bound = (max_kv_len + max_chunk - 1) / max_chunk;
  const long long useful = (max_kv_len + kDecodeMinChunk - 1) / kDecodeMinChunk;
  long long s = fill > bound ? fill : bound;
  if (s > useful) s = useful;
  if (s < 1) s = 1;
  if (s > 65535) s = 65535;
  return (int)s;
}
}  // namespace

int attn_decode_num_splits(int batch, int hkv, int max_kv_len) {
  return split_plan(batch, hkv, max_kv_len, kDecodeTargetWaves, kDecodeMaxChunk);
}

int attn_decode_q4_num_splits(int batch, int hkv, int max_kv_len) {
  return split_plan(batch, hkv, max_kv_len, kDecodeQ4TargetWaves, kDecodeQ4MaxChunk);
}

int attn_decode_chunk_len(int max_kv_len, int num_splits) {
  if (max_kv_len < 1 || num_splits < 1) return 0;
  long long c = ((long long)max_kv_len + num_splits - 1) / num_splits;
  c = (c + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  return (int)c;
}

size_t attn_decode_workspace_bytes(int batch, int hq, int d, int num_splits) {
  if (batch < 1 || hq < 1 || d < 1 || num_splits < 1) return 0;
  return (size_t)batch * hq * num_splits * (size_t)(d + 2) * sizeof(float);
}

attn_status attn_decode_splitk(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                               int max_kv_len, int dtype, int batch, int hq, int hkv, int d, float scale,
                               int num_splits, float* part_m, float* part_l, float* part_o, void* stream) {
  if (!q || !k_cache || !v_cache || !kv_lens || !part_m || !part_l || !part_o) return ATTN_ERR_NULL_PTR;
  if (batch < 1 || hq < 1 || hkv < 1 || max_kv_len < 1 || num_splits < 1 || hq % hkv != 0 || !scale_ok(scale))
    return ATTN_ERR_BAD_SHAPE;
  if ((d != 64 && d != 128) || !dtype_ok(dtype)) return ATTN_ERR_UNSUPPORTED;
  const int groups = (hq / hkv + 15) / 16;
  if ((long long)batch * hkv * max_kv_len * d >= kMaxElems || (long long)max_kv_len * d >= (1LL << 31) ||
      batch > 65535 || (long long)hkv * groups > 65535 || num_splits > 65535 ||
      (long long)batch * hq * num_splits * d >= kMaxElems)
    return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(part_o))
    return ATTN_ERR_MISALIGNED;
  const int chunk = attn_decode_chunk_len(max_kv_len, num_splits);
  return from_hip(attn::launch_decode_splitk(q, k_cache, v_cache, kv_lens, max_kv_len, dtype == ATTN_BF16, batch, hq,
                                             hkv, d, scale, num_splits, chunk, part_m, part_l, part_o,
                                             static_cast<hipStream_t>(stream)));
}

attn_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                                int max_kv_len, int dtype, int batch, int hq, int hkv, int d, float scale,
                                int num_splits, void* o, void* stream) {
  if (!q || !k_cache || !v_cache || !kv_lens || !o) return ATTN_ERR_NULL_PTR;
  if (batch < 1 || hq < 1 || hkv < 1 || max_kv_len < 1 || num_splits < 0 || hq % hkv != 0 || !scale_ok(scale))
    return ATTN_ERR_BAD_SHAPE;
  if ((d != 64 && d != 128) || !dtype_ok(dtype)) return ATTN_ERR_UNSUPPORTED;
  const int S = num_splits > 0 ? num_splits : attn_decode_num_splits(batch, hkv, max_kv_len);
  const int groups = (hq / hkv + 15) / 16;
  if ((long long)batch * hkv * max_kv_len * d >= kMaxElems || (long long)max_kv_len * d >= (1LL << 31) ||
      batch > 65535 || (long long)hkv * groups > 65535 || S > 65535)
    return ATTN_ERR_TOO_LARGE;
  // partials in the scratch array: m [batch, hq, S], l [batch, hq, S], o [batch, hq, S, d], each 256-byte aligned
  const size_t rows = (size_t)batch * hq * S;
  const size_t off_l = align256(rows * sizeof(float));
  const size_t off_o = off_l + align256(rows * sizeof(float));
  if (off_o + rows * (size_t)d * sizeof(float) > ATTN_DECODE_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o)) return ATTN_ERR_MISALIGNED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void* base = nullptr;
  const attn_status s = scratch_address(st, &base);
  if (s != ATTN_OK) return s;
  float* pm = static_cast<float*>(base);
  float* pl = reinterpret_cast<float*>(static_cast<char*>(base) + off_l);
  float* po = reinterpret_cast<float*>(static_cast<char*>(base) + off_o);
  // every partial entry is written by the split-K kernel (an empty split writes (-inf, 0, 0)), so nothing
  // left in the array by an earlier call is read
  const int chunk = attn_decode_chunk_len(max_kv_len, S);
  const hipError_t e = attn::launch_decode_splitk(q, k_cache, v_cache, kv_lens, max_kv_len, dtype == ATTN_BF16,
                                                  batch, hq, hkv, d, scale, S, chunk, pm, pl, po, st);
  if (e != hipSuccess) return ATTN_ERR_LAUNCH;
  return from_hip(attn::launch_merge(pm, pl, po, batch * hq, d, S, dtype == ATTN_BF16, o, st));
}

attn_status attn_decode_splitk_paged(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                                     int max_pages_per_seq, int num_pages, int page_size, const int* kv_lens,
                                     int dtype, int batch, int hq, int hkv, int d, float scale, int num_splits,
                                     int window, const float* alibi_slopes, float* part_m, float* part_l,
                                     float* part_o, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !kv_lens || !part_m || !part_l || !part_o)
    return ATTN_ERR_NULL_PTR;
  if (batch < 1 || hq < 1 || hkv < 1 || max_pages_per_seq < 1 || num_pages < 1 || num_splits < 1 ||
      hq % hkv != 0 || !scale_ok(scale) || window < 0)
    return ATTN_ERR_BAD_SHAPE;
  if (page_size < 16 || (page_size & (page_size - 1)) != 0) return ATTN_ERR_UNSUPPORTED;
  if ((d != 64 && d != 128) || !dtype_ok(dtype)) return ATTN_ERR_UNSUPPORTED;
  const long long max_kv_len = (long long)max_pages_per_seq * page_size;
  const int groups = (hq / hkv + 15) / 16;
  if (max_kv_len * d >= (1LL << 31) || (long long)num_pages * hkv * page_size * d >= kMaxElems ||
      (long long)batch * max_pages_per_seq >= (1LL << 31) || batch > 65535 || (long long)hkv * groups > 65535 ||
      num_splits > 65535 || (long long)batch * hq * num_splits * d >= kMaxElems)
    return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(part_o)) return ATTN_ERR_MISALIGNED;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  const int chunk = attn_decode_chunk_len((int)max_kv_len, num_splits);
  return from_hip(attn::launch_decode_splitk_paged(q, k_pages, v_pages, block_table, max_pages_per_seq, num_pages,
                                                   shift, kv_lens, dtype == ATTN_BF16, batch, hq, hkv, d, scale,
                                                   num_splits, chunk, window, alibi_slopes, part_m, part_l, part_o,
                                                   static_cast<hipStream_t>(stream)));
}

attn_status attn_decode_splitk_q4(const void* q, const void* k_codes, const float* k_scales, const void* v_codes,
                                  const float* v_scales, const int* kv_lens, int max_kv_len, int dtype, int batch,
                                  int hq, int hkv, int d, float scale, int rotated, int num_splits, float* part_m,
                                  float* part_l, float* part_o, void* stream) {
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !kv_lens || !part_m || !part_l || !part_o)
    return ATTN_ERR_NULL_PTR;
  if (batch < 1 || hq < 1 || hkv < 1 || max_kv_len < 1 || num_splits < 1 || hq % hkv != 0 || !scale_ok(scale))
    return ATTN_ERR_BAD_SHAPE;
  if ((d != 64 && d != 128) || !dtype_ok(dtype)) return ATTN_ERR_UNSUPPORTED;
  const int groups = (hq / hkv + 15) / 16;
  if ((long long)batch * hkv * max_kv_len * d >= kMaxElems || (long long)max_kv_len * d >= (1LL << 31) ||
      batch > 65535 || (long long)hkv * groups > 65535 || num_splits > 65535 ||
      (long long)batch * hq * num_splits * d >= kMaxElems)
    return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scales) || !aligned16(v_scales) ||
      !aligned16(part_o))
    return ATTN_ERR_MISALIGNED;
  const int chunk = attn_decode_chunk_len(max_kv_len, num_splits);
  return from_hip(attn::launch_decode_splitk_q4(q, k_codes, k_scales, v_codes, v_scales, kv_lens, max_kv_len,
                                                dtype == ATTN_BF16, batch, hq, hkv, d, scale, rotated != 0, num_splits,
                                                chunk, part_m, part_l, part_o, static_cast<hipStream_t>(stream)));
}

attn_status attn_decode_splitk_q4_paged(const void* q, const void* k_codes, const float* k_scales,
                                        const void* v_codes, const float* v_scales, const int* block_table,
                                        int max_pages_per_seq, int num_pages, int page_size, const int* kv_lens,
                                        int dtype, int batch, int hq, int hkv, int d, float scale, int rotated,
                                        int num_splits, float* part_m, float* part_l, float* part_o, void* stream) {
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !block_table || !kv_lens || !part_m || !part_l ||
      !part_o)
    return ATTN_ERR_NULL_PTR;
  if (batch < 1 || hq < 1 || hkv < 1 || max_pages_per_seq < 1 || num_pages < 1 || num_splits < 1 ||
      hq % hkv != 0 || !scale_ok(scale))
    return ATTN_ERR_BAD_SHAPE;
  if (page_size < 16 || (page_size & (page_size - 1)) != 0) return ATTN_ERR_UNSUPPORTED;
  if ((d != 64 && d != 128) || !dtype_ok(dtype)) return ATTN_ERR_UNSUPPORTED;
  const long long max_kv_len = (long long)max_pages_per_seq * page_size;
  const int groups = (hq / hkv + 15) / 16;
  if (max_kv_len * d >= (1LL << 31) || (long long)num_pages * hkv * page_size * d >= kMaxElems ||
      (long long)batch * max_pages_per_seq >= (1LL << 31) || batch > 65535 || (long long)hkv * groups > 65535 ||
      num_splits > 65535 || (long long)batch * hq * num_splits * d >= kMaxElems)
    return ATTN_ERR_TOO_LARGE;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scales) || !aligned16(v_scales) ||
      !aligned16(part_o))
    return ATTN_ERR_MISALIGNED;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  const int chunk = attn_decode_chunk_len((int)max_kv_len, num_splits);
  return from_hip(attn::launch_decode_splitk_q4_paged(q, k_codes, k_scales, v_codes, v_scales, block_table,
                                                      max_pages_per_seq, num_pages, shift, kv_lens,
                                                      dtype == ATTN_BF16, batch, hq, hkv, d, scale, rotated != 0,
                                                      num_splits, chunk, part_m, part_l, part_o,
                                                      static_cast<hipStream_t>(stream)));
}

attn_status attn_kv_quantize_q4(const void* x, int rows, int d, int dtype, int rotated, const int* out_rows,
                                int out_capacity, void* codes, float* scales, void* stream) {
  if (!x || !codes || !scales) return ATTN_ERR_NULL_PTR;
  if (rows < 1 || out_capacity < 1 || (!out_rows && rows > out_capacity)) return ATTN_ERR_BAD_SHAPE;
  if ((d != 64 && d != 128) || !dtype_ok(dtype)) return ATTN_ERR_UNSUPPORTED;
  if ((long long)rows * d >= kMaxElems || (long long)out_capacity * d >= kMaxElems) return ATTN_ERR_TOO_LARGE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return ATTN_ERR_MISALIGNED;
  const float norm = (float)(1.0 / std::sqrt((double)d));
  return from_hip(attn::launch_quantize_q4(x, rows, d, dtype == ATTN_BF16, rotated != 0, norm, out_rows, out_capacity,
                                           codes, scales, static_cast<hipStream_t>(stream)));
}

attn_status attn_merge_partials(const float* part_m, const float* part_l, const float* part_o, int batch, int hq,
                                int d, int num_splits, void* o, int out_dtype, void* stream) {
  if (!part_m || !part_l || !part_o || !o) return ATTN_ERR_NULL_PTR;
  if (batch < 1 || hq < 1 || num_splits < 1) return ATTN_ERR_BAD_SHAPE;
  if ((d != 64 && d != 128) || !dtype_ok(out_dtype)) return ATTN_ERR_UNSUPPORTED;
  if ((long long)batch * hq * (d / 32) >= (1LL << 31) || (long long)batch * hq * num_splits * d >= kMaxElems)
    return ATTN_ERR_TOO_LARGE;
  if (!aligned16(part_o) || !aligned16(o)) return ATTN_ERR_MISALIGNED;
  return from_hip(attn::launch_merge(part_m, part_l, part_o, batch * hq, d, num_splits, out_dtype == ATTN_BF16, o,
                                     static_cast<hipStream_t>(stream)));
}

attn_status attn_calib_mfma_bf16(float* out, int blocks, int iters, void* stream) {
  if (!out) return ATTN_ERR_NULL_PTR;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24)) return ATTN_ERR_BAD_SHAPE;
  if (!aligned16(out)) return ATTN_ERR_MISALIGNED;
  return from_hip(attn::launch_calib_mfma(out, blocks, iters, static_cast<hipStream_t>(stream)));
}

attn_status attn_calib_read(const void* buf, size_t bytes, void* scratch, int blocks, void* stream) {
  if (!buf || !scratch) return ATTN_ERR_NULL_PTR;
  if (bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20)) return ATTN_ERR_BAD_SHAPE;
  if (!aligned16(buf) || !aligned16(scratch)) return ATTN_ERR_MISALIGNED;
  return from_hip(attn::launch_calib_read(buf, bytes, scratch, blocks, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
