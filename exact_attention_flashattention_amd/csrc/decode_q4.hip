// Split-K single-query decode over a 4-bit KV cache, dequantised inside the
// tile loads ("Why a quantised cache needs a fused kernel" on "Attention from
// the kernel's side"): the kernel reads the 4-bit codes and per-row scales
// straight from HBM and turns them into matrix-core operands in registers, so
// the bytes moved are the quantised cache's and nothing else -- no
// dequantised copy is ever written.
//
// Cache format (one row = one cached position of one KV head, d values):
//   codes  [B, Hkv, Lmax, d/2] bytes: byte i holds elements 2i (low nibble)
//          and 2i+1 (high nibble), each an OCP MX E2M1 code (sign bit 3,
//          exponent bits 2:1, mantissa bit 0; values 0, ±0.5, ±1, ±1.5, ±2,
//          ±3, ±4, ±6);
//   scales [B, Hkv, Lmax] fp32: the row's values are code value × scale.
// With `rotated` the stored rows are R·k and R·v, R = H_d/√d the normalised
// Sylvester-Hadamard matrix (orthogonal and symmetric).  Dot products survive
// the rotation, so the query is rotated once on load and the output rotated
// back once at the end (the rotated-domain trick of the same section).
//
// gfx950 mapping.  The same wave layout as decode_splitk.hip: one wavefront
// per (split, KV head, query group of up to 16 heads, sequence), 32 keys per
// step, the next step's codes and scales in flight while the current ones
// are used.  The codebook is the hardware's: v_cvt_scalef32_pk_{bf16,f16}_fp4
// turns one code byte into two 16-bit operand values in one instruction (its
// scale operand is applied as a power of two only, so it is fed 1.0), and
// the fp32 row scales are applied exactly where they factor out -- the K
// scale multiplies the row's score, the V scale its probability -- instead
// of per element.  The head-dimension order inside an MFMA k-step is free
// (it only has to agree between K and the query), so each lane takes 32
// consecutive dimensions (16 at d=64) and reads its K codes with one 16-byte
// (8-byte) load.  V is dequantised into wave-private LDS in natural order and
// read back with the transpose read as in the 16-bit kernel.
//
// Paged caches (PAGED = true; "PagedAttention's kernel difference" in
// section 5 of "Attention Computation in Practice"): the codes live in a pool
// [num_pages, Hkv, P, d/2] and the scales in [num_pages, Hkv, P]; logical row
// j of sequence b is row j % P of page block_table[b][j / P].  P is a power
// of two >= 16 and splits start on multiples of 64, so each 16-row half of a
// 32-key step lies in one page and gathers through its own buffer resources.
// The V codes are then loaded per half (lane l: row 16·half + l/4, a quarter
// of it) instead of two lanes per row across the step; they land in LDS in
// the same natural order.  The page ids of the split's next 64 pages sit one
// per lane in a VGPR and are picked out with v_readlane.
//
// The P·V product runs in bf16 whatever the query's type: its B operand is a
// probability (up to 2^8 before the reference is raised) times the V row's
// scale, which for legal fp16 V rows (|v| up to 65504, scale up to ~1.1e4)
// would overflow fp16; E2M1 values are exact in bf16, and bf16 has fp32's
// range.
#include "device_common.hpp"
#include "launchers.hpp"

#include <type_traits>

namespace attn {

namespace {

constexpr int kQStep = 32;  // keys per step
constexpr int kQDepth = 2;  // steps in the load ring
constexpr float kQSlack = 8.f;  // log2 of the largest probability used without raising the reference

template <class T>
struct Fp4;
template <>
struct Fp4<Bf16> {
  // the two E2M1 values of byte `sel` of x, as a packed pair (low nibble first)
  static __device__ __forceinline__ uint32_t pair(uint32_t x, int sel);
};
template <>
struct Fp4<F16> {
  static __device__ __forceinline__ uint32_t pair(uint32_t x, int sel);
};
// (the byte selector must be a compile-time constant: one instruction per byte)
#define ATTN_FP4_PAIR(T, FN)                                                                      \
  __device__ __forceinline__ uint32_t Fp4<T>::pair(uint32_t x, int sel) {                         \
    switch (sel) {                                                                                \
      case 0: return __builtin_bit_cast(uint32_t, FN(x, 1.0f, 0));                                \
      case 1: return __builtin_bit_cast(uint32_t, FN(x, 1.0f, 1));                                \
      case 2: return __builtin_bit_cast(uint32_t, FN(x, 1.0f, 2));                                \
      default: return __builtin_bit_cast(uint32_t, FN(x, 1.0f, 3));                               \
    }                                                                                             \
  }
ATTN_FP4_PAIR(Bf16, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4)
ATTN_FP4_PAIR(F16, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4)
#undef ATTN_FP4_PAIR

// 8 code bytes (a u32x2) -> 16 values = two MFMA operands' worth of 8
template <class T>
__device__ __forceinline__ void dequant8(u32x2 c, u32x4& lo, u32x4& hi) {
  lo = u32x4{Fp4<T>::pair(c[0], 0), Fp4<T>::pair(c[0], 1), Fp4<T>::pair(c[0], 2), Fp4<T>::pair(c[0], 3)};
  hi = u32x4{Fp4<T>::pair(c[1], 0), Fp4<T>::pair(c[1], 1), Fp4<T>::pair(c[1], 2), Fp4<T>::pair(c[1], 3)};
}

// One butterfly stage of the Walsh-Hadamard transform across lanes l and
// l ^ 16 (XOR32 = false) or l ^ 32 (true): the lane whose bit is clear keeps
// a + b, its partner a - b (a = the clear lane's value).
template <bool XOR32>
__device__ __forceinline__ float wht_cross(float x, bool upper) {
  const auto r = XOR32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                       : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return upper ? a - b : a + b;
}

// In-lane Walsh-Hadamard stages over the index bits of an array of N values.
template <int N>
__device__ __forceinline__ void wht_inlane(float* x) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
}

template <int D>
struct Q4Stage {
  static constexpr int KB = D / 8;   // code bytes per lane per 16-key half (its D/4 dimensions)
  static constexpr int VB = D / 4;   // V code bytes per lane per step (32 rows · D/2 bytes / 64 lanes)
  u32x4 k[2][KB / 16 > 0 ? KB / 16 : 1];  // d=128: one 16-byte load per half
  u32x2 k8[2];                            // d=64: one 8-byte load per half
  u32x4 v[VB / 16];
  f32x4 ks[2], vs[2];                     // scales of this lane's 4 keys in each half
};

}  // namespace

template <class T, int D, bool PAGED>
// Two waves per SIMD (the register budget of each is 256): the 4-bit steps are
// small, and a second wave per SIMD hides the memory latency that one wave,
// even with four steps in flight, leaves exposed (measured: 79 -> 58 us on a
// 262144-position cache; three waves per SIMD spill and are slower).
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_q4_kernel(
    const char* __restrict__ q, const char* __restrict__ kc, const float* __restrict__ ks,
    const char* __restrict__ vc, const float* __restrict__ vs, const int* __restrict__ kv_lens, int max_kv_len,
    int hq, int hkv, int g, int chunk, int num_splits, float c, int rotated, float* __restrict__ part_m,
    float* __restrict__ part_l, float* __restrict__ part_o, const int* __restrict__ table, int max_pages,
    int num_pages, int page_shift) {
  constexpr int KK = D / 32;             // 16x16x32 k-steps over the head dimension
  constexpr int DG = D / 4;              // dimensions per lane group
  constexpr int DT = D / 16;             // 16-row output tiles of the head dimension
  constexpr int RB = D / 2;              // code bytes per row
  constexpr int VP = 2 * D + 64;         // LDS pitch of a dequantised V row in bytes
  constexpr int VB = Q4Stage<D>::VB;
  __shared__ __attribute__((aligned(16))) char vlds[kQStep * VP];

  const int lane = threadIdx.x;
  const int r = lane & 15;
  const int grp = lane >> 4;
  const int kh = blockIdx.y % hkv;
  const int qgrp = blockIdx.y / hkv;
  const int b = blockIdx.z;
  // split index rotated by the head's number, as in decode_splitk.hip (spreads the
  // waves that run together over different offsets of their heads' cache regions).
  // Paged: not rotated, so the KV heads of one split -- whose rows share each page,
  // and whose scales share 128-byte lines when pages are 16 rows -- land on one XCD
  // (workgroups go round-robin to the 8 XCDs; the split count is then a multiple of 8).
  const int split = PAGED ? (int)blockIdx.x
                          : (int)((blockIdx.x + (unsigned)(b * hkv + kh) * 5u) % (unsigned)num_splits);
  const int qi = qgrp * 16 + r;
  const bool qvalid = qi < g;
  const int h = kh * g + (qvalid ? qi : 0);

  int kv_len = kv_lens[b];
  kv_len = kv_len < 0 ? 0 : (kv_len > max_kv_len ? max_kv_len : kv_len);
  const int start = split * chunk;
  const int end = min(start + chunk, kv_len);

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

  // Query operand: lane (query r, group grp) holds dimensions grp·DG .. grp·DG + DG - 1,
  // rotated into the cache's domain if the cache is, as KK operands of 8.  A rotated
  // query is no longer exact in 16 bits, so it is split into a rounded high part and
  // the rounded remainder, and the scores take one MFMA for each (the matrix cores
  // have time to spare in this memory-bound kernel).
  u32x4 qf[KK], qlo[KK];
  {
    float x[DG];
    const char* qp = q + ((size_t)b * hq + h) * D * 2 + grp * DG * 2;
#pragma unroll
    for (int i = 0; i < DG / 8; ++i) {
      const u32x4 w = qvalid ? gload16(qp + 16 * i) : zero4();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u = w[j];
        if constexpr (std::is_same<T, Bf16>::value) {
          x[8 * i + 2 * j] = __uint_as_float(u << 16);
          x[8 * i + 2 * j + 1] = __uint_as_float(u & 0xffff0000u);
        } else {
          const f16x2 p = __builtin_bit_cast(f16x2, u);
          x[8 * i + 2 * j] = (float)p[0];
          x[8 * i + 2 * j + 1] = (float)p[1];
        }
      }
    }
    if (rotated) {  // x <- H_D x / sqrt(D): in-lane over the low index bits, across lane groups for the top two
      wht_inlane<DG>(x);
      const float inv_sqrt = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
      for (int i = 0; i < DG; ++i) {
        x[i] = wht_cross<false>(x[i], grp & 1);
        x[i] = wht_cross<true>(x[i], grp & 2) * inv_sqrt;
      }
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      float rem[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t hi = T::pack2(x[8 * kk + 2 * j], x[8 * kk + 2 * j + 1]);
        qf[kk][j] = hi;
        float h0, h1;
        if constexpr (std::is_same<T, Bf16>::value) {
          h0 = __uint_as_float(hi << 16);
          h1 = __uint_as_float(hi & 0xffff0000u);
        } else {
          const f16x2 p = __builtin_bit_cast(f16x2, hi);
          h0 = (float)p[0];
          h1 = (float)p[1];
        }
        rem[2 * j] = x[8 * kk + 2 * j] - h0;
        rem[2 * j + 1] = x[8 * kk + 2 * j + 1] - h1;
      }
      qlo[kk] = u32x4{T::pack2(rem[0], rem[1]), T::pack2(rem[2], rem[3]), T::pack2(rem[4], rem[5]),
                      T::pack2(rem[6], rem[7])};
    }
  }

  const size_t head = (size_t)b * hkv + kh;
  const char* kbase = kc + head * (size_t)max_kv_len * RB;
  const char* vbase = vc + head * (size_t)max_kv_len * RB;
  const float* ksbase = ks + head * (size_t)max_kv_len;
  const float* vsbase = vs + head * (size_t)max_kv_len;

  // per-lane byte offsets within a step (fixed; each step moves the scalar bases)
  const uint32_t k_off = (uint32_t)r * RB + grp * (DG / 2);             // + 16·sb·RB for half sb
  const uint32_t s_off = (uint32_t)(4 * grp) * 4;                       // + 64·sb for half sb
  const int vrow = lane / (64 / 32);                                    // V rows: two lanes per row
  const uint32_t v_off = (uint32_t)vrow * RB + (lane & 1) * (RB / 2);   // VB = RB/2 bytes per lane
  // paged: V loaded per 16-row half, lane l taking row l/4 of the half, quarter l%4 of it
  const uint32_t pv_off = (uint32_t)(lane >> 2) * RB + (lane & 3) * (RB / 4);

  // paged: ids of pages [tab_base, tab_base + 64) of this sequence, lane i
  // holding page tab_base + i (entries past the table row read as 0)
  int tab = 0, tab_base = 0;
  auto fetch_table = [&](int p0) {
    tab_base = p0;
    const int p = p0 + lane;
    tab = p < max_pages ? table[(size_t)b * max_pages + p] : 0;
  };
  if constexpr (PAGED) fetch_table(start >> page_shift);
  // pool row of logical row `key` (a multiple of 16) of KV head kh
  auto paged_row = [&](int key) -> size_t {
    const int p = key >> page_shift;
    if (p - tab_base >= 64) fetch_table(p);
    int id = __builtin_amdgcn_readlane(tab, p - tab_base);
    id = id < 0 ? 0 : (id >= num_pages ? num_pages - 1 : id);
    return (((size_t)id * hkv + kh) << page_shift) + (key & ((1 << page_shift) - 1));
  };

  auto load = [&](Q4Stage<D>& st, int k0) {
    if constexpr (PAGED) {
      bufres rk[2], rv[2], rks[2], rvs[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kr = k0 + 16 * sb;
        // (readfirstlane: a resource in vector registers would make every load a waterfall loop)
        const int rows = __builtin_amdgcn_readfirstlane(end - kr < 0 ? 0 : (end - kr > 16 ? 16 : end - kr));
        const size_t row = rows > 0 ? paged_row(kr) : 0;  // past the end: reads nothing
        rk[sb] = make_bufres(kc + row * RB, (uint32_t)rows * RB);
        rv[sb] = make_bufres(vc + row * RB, (uint32_t)rows * RB);
        rks[sb] = make_bufres(ks + row, (uint32_t)rows * 4);
        rvs[sb] = make_bufres(vs + row, (uint32_t)rows * 4);
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if constexpr (D == 128) {
          st.k[sb][0] = bload16(rk[sb], k_off);
          st.v[sb] = bload16(rv[sb], pv_off);
        } else {
          st.k8[sb] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk[sb], k_off, 0, 0));
          const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv[sb], pv_off, 0, 0));
          st.v[0][2 * sb] = w[0];
          st.v[0][2 * sb + 1] = w[1];
        }
        st.ks[sb] = __builtin_bit_cast(f32x4, bload16(rks[sb], s_off));
        st.vs[sb] = __builtin_bit_cast(f32x4, bload16(rvs[sb], s_off));
      }
      return;
    }
    const uint32_t rows = k0 < end ? (uint32_t)(end - k0) : 0u;  // past the end: reads nothing
    const bufres rk = make_bufres(kbase + (size_t)k0 * RB, rows * RB);
    const bufres rv = make_bufres(vbase + (size_t)k0 * RB, rows * RB);
    const bufres rks = make_bufres(ksbase + k0, rows * 4);
    const bufres rvs = make_bufres(vsbase + k0, rows * 4);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      if constexpr (D == 128) {
        st.k[sb][0] = bload16(rk, k_off + sb * 16 * RB);
      } else {
        st.k8[sb] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, k_off + sb * 16 * RB, 0, 0));
      }
      st.ks[sb] = __builtin_bit_cast(f32x4, bload16(rks, s_off + sb * 64));
      st.vs[sb] = __builtin_bit_cast(f32x4, bload16(rvs, s_off + sb * 64));
    }
#pragma unroll
    for (int i = 0; i < VB / 16; ++i) st.v[i] = bload16(rv, v_off + 16 * i);
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const Q4Stage<D>& st, int k0) {
    __syncthreads();  // previous step's transpose reads are done with the buffer
    // V codes -> 16-bit values in LDS, natural dimension order: this lane's VB bytes
    // are dimensions (lane & 1)·D/2 .. + D/2 - 1 of row vrow (paged: per half h,
    // dimensions (lane & 3)·D/4 .. + D/4 - 1 of row 16·h + lane/4)
    if constexpr (PAGED) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint32_t at = (16 * h2 + (lane >> 2)) * VP + (lane & 3) * (D / 2);
        u32x4 lo, hi;
        if constexpr (D == 128) {
          dequant8<Bf16>(u32x2{st.v[h2][0], st.v[h2][1]}, lo, hi);
          lds_write16(vlds, at, lo);
          lds_write16(vlds, at + 16, hi);
          dequant8<Bf16>(u32x2{st.v[h2][2], st.v[h2][3]}, lo, hi);
          lds_write16(vlds, at + 32, lo);
          lds_write16(vlds, at + 48, hi);
        } else {
          dequant8<Bf16>(u32x2{st.v[0][2 * h2], st.v[0][2 * h2 + 1]}, lo, hi);
          lds_write16(vlds, at, lo);
          lds_write16(vlds, at + 16, hi);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < VB / 16; ++i) {
        u32x4 lo, hi;
        dequant8<Bf16>(u32x2{st.v[i][0], st.v[i][1]}, lo, hi);
        const uint32_t at = vrow * VP + (lane & 1) * D + i * 64;
        lds_write16(vlds, at, lo);
        lds_write16(vlds, at + 16, hi);
        dequant8<Bf16>(u32x2{st.v[i][2], st.v[i][3]}, lo, hi);
        lds_write16(vlds, at + 32, lo);
        lds_write16(vlds, at + 48, hi);
      }
    }
    // scores: s[sb][e] is key k0 + 16·sb + 4·grp + e against query column r
    f32x4 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      u32x4 kf[KK];
      if constexpr (D == 128) {
        dequant8<T>(u32x2{st.k[sb][0][0], st.k[sb][0][1]}, kf[0], kf[1]);
        dequant8<T>(u32x2{st.k[sb][0][2], st.k[sb][0][3]}, kf[2], kf[3]);
      } else {
        dequant8<T>(st.k8[sb], kf[0], kf[1]);
      }
      s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) s[sb] = T::mfma16(kf[kk], qf[kk], s[sb]);
      if (rotated) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s[sb] = T::mfma16(kf[kk], qlo[kk], s[sb]);
      }
      s[sb] *= st.ks[sb];  // the K rows' scales
    }
    if (k0 + kQStep > end) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (k0 + sb * 16 + 4 * grp + e >= end) s[sb][e] = kNegInf;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = max_xor32(max_xor16(mx)) * c;
    // The exponentials use the reference m_run, raised (with l and o rescaled by
    // exp2(m_run - m_new)) only when some row's maximum passes it by more than
    // 2^8; probabilities stay below 2^8 and o/l is unchanged, while the output
    // rescale leaves the common path.  Every processed step holds a live key,
    // so the first step sets a finite reference.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kQSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);  // 0 on the first step
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(fmaf(s[sb][e], c, -m_run));
        psum += p;
        s[sb][e] = p * st.vs[sb][e];  // the V row's scale rides on its probability
      }
    l_run += psum;
    const u32x4 pf = {Bf16::pack2(s[0][0], s[0][1]), Bf16::pack2(s[0][2], s[0][3]), Bf16::pack2(s[1][0], s[1][1]),
                      Bf16::pack2(s[1][2], s[1][3])};
    __syncthreads();  // V rows are in LDS
    const uint32_t row_a = (4 * grp + (r >> 2)) * VP;
    const uint32_t row_b = (16 + 4 * grp + (r >> 2)) * VP;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t col = (dt * 16 + 4 * (r & 3)) * 2;
      const u32x2 va = lds_read_tr16(vlds, row_a + col);
      const u32x2 vb = lds_read_tr16(vlds, row_b + col);
      oacc[dt] = Bf16::mfma16(u32x4{va[0], va[1], vb[0], vb[1]}, pf, oacc[dt]);
    }
  };

  // A ring of kQDepth steps: while step i is processed, steps i+1 .. i+kQDepth-1
  // are in flight.  With 2048 waves of eight small loads per step the memory
  // pipeline, not the latency, sets the pace: one step ahead reads the cache
  // faster than three (measured on 262144 positions: 4.5 against 4.3 TB/s by
  // wall clock with the merge) and needs 66 fewer registers.
  // The loads are issued unconditionally (past the end they read nothing), so
  // the compiler can count the steps in flight and wait for the current one only.
  Q4Stage<D> st[kQDepth];
#pragma unroll
  for (int i = 0; i + 1 < kQDepth; ++i) load(st[i], start + i * kQStep);
  bool done = false;
  for (int k0 = start; !done; k0 += kQDepth * kQStep) {
#pragma unroll
    for (int i = 0; i < kQDepth; ++i) {
      const int ahead = k0 + (i + kQDepth - 1) * kQStep;
      load(st[(i + kQDepth - 1) % kQDepth], ahead);
      process(st[i], k0 + i * kQStep);
      if (k0 + (i + 1) * kQStep >= end) {
        done = true;
        break;
      }
    }
  }

  // rotate the partial output back: oacc[dt][e] is dimension 16·dt + 4·grp + e
  if (rotated) {
    float x[4 * DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * dt + e] = oacc[dt][e];
    // in-lane index 4·dt + e carries dimension bits 0-1 (e) and 4.. (dt); bits 2-3 are the lane group
    wht_inlane<4 * DT>(x);
    const float inv_sqrt = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
    for (int i = 0; i < 4 * DT; ++i) {
      x[i] = wht_cross<false>(x[i], grp & 1);
      x[i] = wht_cross<true>(x[i], grp & 2) * inv_sqrt;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[dt][e] = x[4 * dt + e];
  }

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

template <class T, int D, bool PAGED>
static hipError_t launch_q4_t(const void* q, const void* kc, const float* ks, const void* vc, const float* vs,
                              const int* kv_lens, int max_kv_len, int batch, int hq, int hkv, float scale, int rotated,
                              int num_splits, int chunk, float* pm, float* pl, float* po, const int* table,
                              int max_pages, int num_pages, int page_shift, hipStream_t stream) {
  const int g = hq / hkv;
  const int groups = (g + 15) / 16;
  dim3 grid(num_splits, hkv * groups, batch);
  decode_q4_kernel<T, D, PAGED><<<grid, dim3(64), 0, stream>>>(
      static_cast<const char*>(q), static_cast<const char*>(kc), ks, static_cast<const char*>(vc), vs, kv_lens,
      max_kv_len, hq, hkv, g, chunk, num_splits, scale * kLog2e, rotated, pm, pl, po, table, max_pages, num_pages,
      page_shift);
  return hipGetLastError();
}

template <bool PAGED>
static hipError_t launch_q4_any(const void* q, const void* kc, const float* ks, const void* vc, const float* vs,
                                const int* kv_lens, int max_kv_len, bool bf16, int batch, int hq, int hkv, int d,
                                float scale, bool rotated, int num_splits, int chunk, float* pm, float* pl, float* po,
                                const int* table, int max_pages, int num_pages, int page_shift, hipStream_t stream) {
  const int rot = rotated ? 1 : 0;
  if (bf16)
    return d == 64 ? launch_q4_t<Bf16, 64, PAGED>(q, kc, ks, vc, vs, kv_lens, max_kv_len, batch, hq, hkv, scale, rot,
                                                  num_splits, chunk, pm, pl, po, table, max_pages, num_pages,
                                                  page_shift, stream)
                   : launch_q4_t<Bf16, 128, PAGED>(q, kc, ks, vc, vs, kv_lens, max_kv_len, batch, hq, hkv, scale, rot,
                                                   num_splits, chunk, pm, pl, po, table, max_pages, num_pages,
                                                   page_shift, stream);
  return d == 64 ? launch_q4_t<F16, 64, PAGED>(q, kc, ks, vc, vs, kv_lens, max_kv_len, batch, hq, hkv, scale, rot,
                                               num_splits, chunk, pm, pl, po, table, max_pages, num_pages, page_shift,
                                               stream)
                 : launch_q4_t<F16, 128, PAGED>(q, kc, ks, vc, vs, kv_lens, max_kv_len, batch, hq, hkv, scale, rot,
                                                num_splits, chunk, pm, pl, po, table, max_pages, num_pages,
                                                page_shift, stream);
}

hipError_t launch_decode_splitk_q4(const void* q, const void* k_codes, const float* k_scales, const void* v_codes,
                                   const float* v_scales, const int* kv_lens, int max_kv_len, bool bf16, int batch,
                                   int hq, int hkv, int d, float scale, bool rotated, int num_splits, int chunk,
                                   float* part_m, float* part_l, float* part_o, hipStream_t stream) {
  return launch_q4_any<false>(q, k_codes, k_scales, v_codes, v_scales, kv_lens, max_kv_len, bf16, batch, hq, hkv, d,
                              scale, rotated, num_splits, chunk, part_m, part_l, part_o, nullptr, 0, 0, 0, stream);
}

hipError_t launch_decode_splitk_q4_paged(const void* q, const void* k_codes, const float* k_scales,
                                         const void* v_codes, const float* v_scales, const int* block_table,
                                         int max_pages, int num_pages, int page_shift, const int* kv_lens, bool bf16,
                                         int batch, int hq, int hkv, int d, float scale, bool rotated, int num_splits,
                                         int chunk, float* part_m, float* part_l, float* part_o, hipStream_t stream) {
  return launch_q4_any<true>(q, k_codes, k_scales, v_codes, v_scales, kv_lens, max_pages << page_shift, bf16, batch,
                             hq, hkv, d, scale, rotated, num_splits, chunk, part_m, part_l, part_o, block_table,
                             max_pages, num_pages, page_shift, stream);
}

}  // namespace attn
