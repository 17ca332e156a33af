// Split-K single-query decode: partial (m, l, o) states per slice of the KV
// cache ("Flash-Decoding": the cache sequence is split across workgroups so
// one query per sequence still fills the GPU -- "Prefill and decode are
// different problems" on "Attention from the kernel's side", and "The four
// attention kernels you actually use" in section 5 of "Attention Computation
// in Practice").  The partials are merged by merge_partials.hip.
//
// Work decomposition: one wavefront per (split, KV head, query group,
// sequence).  A query group is up to 16 of the g = hq/hkv query heads that
// share the KV head, so every K/V byte the wave streams is used by all of
// them (GQA reuse, "GQA in the kernel").  The wave walks its slice 32 keys at
// a time; the next 32 keys' K and V rows are already in flight (16-byte
// buffer loads into registers, clipped to the sequence's length) while the
// current ones are used:
//
//   scores   Sᵀ[32 keys × 16 queries] = K·Qᵀ on 16x16x32 MFMA, K straight
//            from its registers, Q resident in registers;
//   softmax  running max / sum per query column, rescale by exp2(m − m_new)
//            (the online recurrence of "The online softmax"), scores held in
//            the exp2 domain (scale·log2 e folded into one FMA);
//   values   V rows go to a wave-private LDS buffer and come back through the
//            LDS transpose read as the k-major A operand of
//            Oᵀ[D × 16] += Vᵀ·Pᵀ, P rounded to the storage type.
//
// The kernel is bound by HBM reads of K and V; the matrix cores and the
// softmax arithmetic are far below their limits at g <= 16.
//
// Paged caches ("PagedAttention's kernel difference" in section 5 of
// "Attention Computation in Practice"): the same kernel with PAGED = true
// reads logical cache row j of sequence b from page block_table[b][j / P] at
// row j % P, the pool laid out [num_pages, hkv, P, d].  P is a power of two
// >= 16 and every split starts on a multiple of 64, so each 16-row half of a
// 32-key step lies inside one page: a step gathers through two buffer
// resources per tensor instead of one.  The page ids of the split's next 64
// pages sit one per lane in a VGPR (one vector load, refreshed when a split
// runs past them) and are picked out with v_readlane, so the gather adds no
// memory round trip to a step.
//
// The paged kernel also takes the masking variants of "Masking variants"
// (same section), for the query at position p = kv_len - 1: a sliding window
// W keeps keys p - W < j <= p (splits wholly before the window are empty, the
// others start at the first 32-key step the window reaches), and ALiBi adds
// -m_h·(p - j) to every score of query head h, folded into the raw scores as
// (m_h / scale)·(j - p).
#include "device_common.hpp"
#include "launchers.hpp"

namespace attn {

namespace {

constexpr int kStep = 32;  // keys per step

template <int D>
struct DecodeStage {
  static constexpr int KK = D / 32;        // 16x16x32 k-steps over the head dimension
  static constexpr int VCH = D / 16;       // 16-byte V chunks per lane per step (32 rows · D/8 chunks / 64)
  u32x4 k[2][KK];                          // [key subtile][k-step]
  u32x4 v[VCH];
};

}  // namespace

// Where a paged kernel finds its pages (unused by the contiguous kernel).
struct PageTable {
  const int* table;  // [batch, max_pages] page ids
  int max_pages;     // table row length
  int num_pages;     // pages in the pool; ids are clamped into [0, num_pages)
  int shift;         // log2 of the page size
};

// Masking variants of the paged kernel (zero / null: none).
struct DecodeMask {
  int window;          // > 0: only the last `window` keys are visible
  const float* alibi;  // [hq] ALiBi slopes, natural-log units per position
};

template <class T, int D, bool PAGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_splitk_kernel(
    const char* __restrict__ q, const char* __restrict__ kc, const char* __restrict__ vc,
    const int* __restrict__ kv_lens, int max_kv_len, int hq, int hkv, int g, int chunk, int num_splits, float c,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ part_o, PageTable pt,
    DecodeMask mk) {
  constexpr int KK = D / 32;
  constexpr int DT = D / 16;              // 16-row output tiles of the head dimension
  constexpr int VCH = D / 16;
  constexpr int VP = 2 * D + 64;          // LDS pitch of a V row in bytes (bank-spread for the transpose read)
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  __shared__ __attribute__((aligned(16))) char vlds[kStep * VP];

  const int lane = threadIdx.x;
  const int r = lane & 15;                // MFMA column: query within the group / row within a tile
  const int grp = lane >> 4;              // lane group 0..3
  const int kh = blockIdx.y % hkv;
  const int qgrp = blockIdx.y / hkv;
  const int b = blockIdx.z;
  // Blocks of one (sequence, KV head) are dispatched together; rotating their
  // split index by the head's number puts the waves that run at the same time
  // at different offsets of their heads' cache regions.  With power-of-two
  // region sizes and ragged lengths, unrotated waves of many heads read the
  // same offsets at once and contend for the same DRAM banks (measured on 64
  // ragged sequences in a 32768-position cache: 4.4 -> 5.35 TB/s).
  const int split = (int)((blockIdx.x + (unsigned)(b * hkv + kh) * 5u) % (unsigned)num_splits);
  const int qi = qgrp * 16 + r;           // query index within the KV head's group
  const bool qvalid = qi < g;
  const int h = kh * g + (qvalid ? qi : 0);

  int kv_len = kv_lens[b];
  kv_len = kv_len < 0 ? 0 : (kv_len > max_kv_len ? max_kv_len : kv_len);
  // first visible key: 0, or the window's first key; a split starts at the
  // first 32-key step that holds a visible key
  const int lo = (PAGED && mk.window > 0) ? max(0, kv_len - mk.window) : 0;
  const int start = PAGED ? max(split * chunk, lo & ~(kStep - 1)) : split * chunk;
  const int end = min(split * chunk + chunk, kv_len);

  const size_t prow = ((size_t)b * hq + h) * num_splits + split;
  float* po = part_o + prow * D;

  if (start >= end) {  // no keys in this slice: the empty state (-inf, 0, 0)
    if (qvalid) {
      if (grp == 0) {
        part_m[prow] = kNegInf;
        part_l[prow] = 0.f;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16 + 4 * grp) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }

  // Q operand (B of Sᵀ = K·Qᵀ): lane (query r, group grp) holds d-chunk 4·kk + grp.
  u32x4 qf[KK];
  {
    const char* qp = q + ((size_t)b * hq + h) * D * 2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = qvalid ? gload16(qp + (4 * kk + grp) * 16) : zero4();
  }

  const size_t head_base = ((size_t)b * hkv + kh) * (size_t)max_kv_len * D * 2;
  const char* kbase = kc + head_base;
  const char* vbase = vc + head_base;

  // Loads go through buffer resources that cover rows [k0, end) only: rows at
  // or past the sequence's length read as 0 and are never touched in memory.
  // The per-lane offsets are fixed; each step only moves the scalar base.
  uint32_t k_off[2][KK], v_off[VCH];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) k_off[sb][kk] = (uint32_t)(sb * 16 + r) * D * 2 + (4 * kk + grp) * 16;
#pragma unroll
  for (int i = 0; i < VCH; ++i) {
    const int cidx = lane + 64 * i;
    v_off[i] = (uint32_t)(cidx / CPR) * D * 2 + (cidx % CPR) * 16;
  }
  // paged: ids of pages [tab_base, tab_base + 64) of this sequence, lane i
  // holding page tab_base + i (entries past the table row read as 0)
  int tab = 0, tab_base = 0;
  auto fetch_table = [&](int p0) {
    tab_base = p0;
    const int p = p0 + lane;
    tab = p < pt.max_pages ? pt.table[(size_t)b * pt.max_pages + p] : 0;
  };
  if constexpr (PAGED) fetch_table(start >> pt.shift);
  // byte offset in the pool of logical row `key` (a multiple of 16) of KV head kh
  auto paged_row = [&](int key) -> size_t {
    const int p = key >> pt.shift;
    if (p - tab_base >= 64) fetch_table(p);
    int id = __builtin_amdgcn_readlane(tab, p - tab_base);
    id = id < 0 ? 0 : (id >= pt.num_pages ? pt.num_pages - 1 : id);
    return ((((size_t)id * hkv + kh) << pt.shift) + (key & ((1 << pt.shift) - 1))) * (size_t)(D * 2);
  };

  auto load = [&](DecodeStage<D>& st, int k0) {
    if constexpr (PAGED) {
      // rows [k0 + 16·sb, +16) of each half lie in one page
      constexpr int VHALF = VCH / 2;  // V chunks per 16-row half
      bufres rk[2], rv[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kr = k0 + 16 * sb;
        // (readfirstlane: the clamp may be computed with a vector min/max, and a
        // resource in vector registers would make every load a waterfall loop)
        const int rows = __builtin_amdgcn_readfirstlane(end - kr < 0 ? 0 : (end - kr > 16 ? 16 : end - kr));
        const size_t off = rows > 0 ? paged_row(kr) : 0;
        rk[sb] = make_bufres(kc + off, (uint32_t)rows * D * 2);
        rv[sb] = make_bufres(vc + off, (uint32_t)rows * D * 2);
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) st.k[sb][kk] = bload16(rk[sb], k_off[0][kk]);
#pragma unroll
      for (int i = 0; i < VCH; ++i)
        st.v[i] = bload16(rv[i / VHALF], v_off[i] - (uint32_t)(i / VHALF) * 16 * D * 2);
    } else {
      const uint32_t bytes = k0 < end ? (uint32_t)(end - k0) * D * 2 : 0u;  // past the end: reads nothing
      const bufres rk = make_bufres(kbase + (size_t)k0 * D * 2, bytes);
      const bufres rv = make_bufres(vbase + (size_t)k0 * D * 2, bytes);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) st.k[sb][kk] = bload16(rk, k_off[sb][kk]);
#pragma unroll
      for (int i = 0; i < VCH; ++i) st.v[i] = bload16(rv, v_off[i]);
    }
  };

  // ALiBi slope of this lane's query head in raw-score units (scores are scaled by c = scale·log2 e later)
  const float alibi_raw = (PAGED && mk.alibi != nullptr && qvalid) ? mk.alibi[h] * kLog2e / c : 0.f;
  const bool alibi = PAGED && mk.alibi != nullptr;

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const DecodeStage<D>& st, int k0) {
    __syncthreads();  // previous step's transpose reads are done with the buffer
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int cidx = lane + 64 * i;
      lds_write16(vlds, (cidx / CPR) * VP + (cidx % CPR) * 16, st.v[i]);
    }
    // scores: s[sb][e] is key k0 + 16·sb + 4·grp + e against query column r
    f32x4 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) s[sb] = T::mfma16(st.k[sb][kk], qf[kk], s[sb]);
    }
    if (alibi) {  // + (m/scale)·(j - p) for key j = k0 + 16·sb + 4·grp + e, p = kv_len - 1
      const float base = alibi_raw * (float)(k0 + 4 * grp - (kv_len - 1));
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[sb][e] += fmaf(alibi_raw, (float)(16 * sb + e), base);
    }
    if (k0 + kStep > end || (PAGED && k0 < lo)) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + sb * 16 + 4 * grp + e;
          if (key >= end || (PAGED && key < lo)) s[sb][e] = kNegInf;
        }
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = max_xor32(max_xor16(mx));
    // every processed step holds at least one live key (a split starts at or
    // after the step holding lo), so m_new is finite
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);  // 0 on the first step (m_run = -inf)
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(fmaf(s[sb][e], c, -m_new));
        s[sb][e] = p;
        psum += p;
      }
    l_run = fmaf(l_run, alpha, psum);
    m_run = m_new;
    const u32x4 pf = {T::pack2(s[0][0], s[0][1]), T::pack2(s[0][2], s[0][3]), T::pack2(s[1][0], s[1][1]),
                      T::pack2(s[1][2], s[1][3])};
    __syncthreads();  // V rows are in LDS
    const uint32_t row_a = (4 * grp + (r >> 2)) * VP;
    const uint32_t row_b = (16 + 4 * grp + (r >> 2)) * VP;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t col = (dt * 16 + 4 * (r & 3)) * 2;
      const u32x2 va = lds_read_tr16(vlds, row_a + col);
      const u32x2 vb = lds_read_tr16(vlds, row_b + col);
      oacc[dt] = T::mfma16(u32x4{va[0], va[1], vb[0], vb[1]}, pf, oacc[dt] * alpha);
    }
  };

  // The next step's loads are issued unconditionally (past the end they read
  // nothing): with a conditional load the compiler cannot count the loads in
  // flight and waits for all of them, the next step's included, before using
  // the current step's registers.
  DecodeStage<D> A, B;
  load(A, start);
  for (int k0 = start;; k0 += 2 * kStep) {
    load(B, k0 + kStep);
    process(A, k0);
    if (k0 + kStep >= end) break;
    load(A, k0 + 2 * kStep);
    process(B, k0 + kStep);
    if (k0 + 2 * kStep >= end) break;
  }

  // partial state of this slice, natural-log units
  const float l_tot = sum_xor32(sum_xor16(l_run));
  if (qvalid) {
    if (grp == 0) {
      part_m[prow] = m_run * kLn2;
      part_l[prow] = l_tot;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16 + 4 * grp) = oacc[dt];
  }
}

// LDS reserved by every decode workgroup beside its own small buffer, so that
// at most two of them (two waves) share a compute unit: gfx950 has 160 KB of
// LDS per CU and a workgroup then takes 64 KB + its ~10 KB.  Fewer concurrent
// cache streams read HBM faster -- on 64 ragged sequences of up to 32768 keys
// 5.84 TB/s against 5.60 with up to four per CU (one per SIMD), and one per CU
// is too few (5.0); a single long sequence, whose 512 waves sit two per CU
// anyway, is unchanged (measured).
constexpr unsigned kDecodeLdsReserve = 64u * 1024u;

template <class T, int D, bool PAGED>
static hipError_t launch_decode_t(const void* q, const void* kc, const void* vc, const int* kv_lens, int max_kv_len,
                                  int batch, int hq, int hkv, float scale, int num_splits, int chunk, float* pm,
                                  float* pl, float* po, PageTable pt, DecodeMask mk, hipStream_t stream) {
  const int g = hq / hkv;
  const int groups = (g + 15) / 16;
  dim3 grid(num_splits, hkv * groups, batch);
  decode_splitk_kernel<T, D, PAGED><<<grid, dim3(64), kDecodeLdsReserve, stream>>>(
      static_cast<const char*>(q), static_cast<const char*>(kc), static_cast<const char*>(vc), kv_lens, max_kv_len,
      hq, hkv, g, chunk, num_splits, scale * kLog2e, pm, pl, po, pt, mk);
  return hipGetLastError();
}

template <bool PAGED>
static hipError_t launch_decode_any(const void* q, const void* kc, const void* vc, const int* kv_lens,
                                    int max_kv_len, bool bf16, int batch, int hq, int hkv, int d, float scale,
                                    int num_splits, int chunk, float* pm, float* pl, float* po, PageTable pt,
                                    DecodeMask mk, hipStream_t stream) {
  if (bf16) {
    return d == 64 ? launch_decode_t<Bf16, 64, PAGED>(q, kc, vc, kv_lens, max_kv_len, batch, hq, hkv, scale,
                                                      num_splits, chunk, pm, pl, po, pt, mk, stream)
                   : launch_decode_t<Bf16, 128, PAGED>(q, kc, vc, kv_lens, max_kv_len, batch, hq, hkv, scale,
                                                       num_splits, chunk, pm, pl, po, pt, mk, stream);
  }
  return d == 64 ? launch_decode_t<F16, 64, PAGED>(q, kc, vc, kv_lens, max_kv_len, batch, hq, hkv, scale,
                                                   num_splits, chunk, pm, pl, po, pt, mk, stream)
                 : launch_decode_t<F16, 128, PAGED>(q, kc, vc, kv_lens, max_kv_len, batch, hq, hkv, scale,
                                                    num_splits, chunk, pm, pl, po, pt, mk, stream);
}

hipError_t launch_decode_splitk(const void* q, const void* k_cache, const void* v_cache, const int* kv_lens,
                                int max_kv_len, bool bf16, int batch, int hq, int hkv, int d, float scale,
                                int num_splits, int chunk, float* part_m, float* part_l, float* part_o,
                                hipStream_t stream) {
  return launch_decode_any<false>(q, k_cache, v_cache, kv_lens, max_kv_len, bf16, batch, hq, hkv, d, scale,
                                  num_splits, chunk, part_m, part_l, part_o, PageTable{nullptr, 0, 0, 0},
                                  DecodeMask{0, nullptr}, stream);
}

hipError_t launch_decode_splitk_paged(const void* q, const void* k_pages, const void* v_pages,
                                      const int* block_table, int max_pages, int num_pages, int page_shift,
                                      const int* kv_lens, bool bf16, int batch, int hq, int hkv, int d, float scale,
                                      int num_splits, int chunk, int window, const float* alibi, float* part_m,
                                      float* part_l, float* part_o, hipStream_t stream) {
  return launch_decode_any<true>(q, k_pages, v_pages, kv_lens, max_pages << page_shift, bf16, batch, hq, hkv, d,
                                 scale, num_splits, chunk, part_m, part_l, part_o,
                                 PageTable{block_table, max_pages, num_pages, page_shift}, DecodeMask{window, alibi},
                                 stream);
}

}  // namespace attn
