// Prefill forward: exact attention of a square problem, tile by tile.
//
// FlashAttention as described in "FlashAttention: what never touches memory"
// ("Attention from the kernel's side") and "03 · The structure" ("Quantized
// kernels"): a block of query rows stays resident, tiles of K and V stream
// past it through on-chip memory, each tile's scores update the running
// (m, l, o) of every row with the online-softmax recurrence, and O is written
// once.  Scores and probabilities exist only in registers.
//
// gfx950 mapping (one workgroup = 4 wavefronts = 128 query rows, two
// workgroups per CU so each SIMD runs two waves):
//   * each wave owns 32 query rows; its Q rows sit in registers as the
//     B operand of the 32x32x16 matrix instruction;
//   * K and V tiles of 64 keys are fetched one tile ahead with 16-byte buffer
//     loads (out-of-range rows read as 0, so the tail needs no branches) and
//     stored to a double-buffered LDS stage; the loop is unrolled by two so
//     both stages are addressed with immediate offsets;
//   * scores are computed transposed, Sᵀ = K·Qᵀ, so that each lane holds 16
//     keys of ONE query: the row max needs only an in-lane max plus one
//     exchange between the wave's halves (v_permlane32_swap), the rescale
//     factor is one scalar per lane, and the probabilities are already in
//     the register layout of the B operand of Oᵀ += Vᵀ·Pᵀ (no shuffle);
//   * each 32-key subtile runs scores -> softmax -> P·V on its own, so the
//     next subtile's score MFMAs have no dependence on this subtile's
//     softmax and can issue under it;
//   * V reaches the matrix cores through the LDS transpose read
//     (ds_read_b64_tr_b16), which delivers 4 consecutive keys of one
//     head-dimension column per lane;
//   * the softmax runs in the exp2 domain (scale·log2 e folded into one FMA
//     per score, v_exp_f32); the running maximum is raised only when a row's
//     new maximum exceeds it by more than 2^8 (o and l share the reference, so
//     o/l is unchanged), which keeps the output rescale off the common path;
//   * causal: key tiles wholly above a wave's diagonal are skipped, the mask
//     is applied only on subtiles that cross the diagonal or the sequence end
//     (block classification of "Masking variants", "Attention Computation in
//     Practice" section 5), and the heaviest query tiles are launched first.
#include "device_common.hpp"
#include "launchers.hpp"

namespace attn {

namespace {

// Largest growth of a row maximum (in log2 units) absorbed without rescaling.
constexpr float kRescaleLog2 = 8.f;

template <int D>
struct PrefillCfg {
  static constexpr int WAVES = 4;
  static constexpr int BR = 32 * WAVES;        // query rows per workgroup
  static constexpr int BC = 64;                // keys per tile
  static constexpr int KP = 2 * D + 16;        // LDS pitch of a K row (bytes): 4-bank row skew
  static constexpr int VP = 2 * D + 64;        // LDS pitch of a V row (bytes): 16-bank row skew
  static constexpr int KBYTES = BC * KP;
  static constexpr int VBYTES = BC * VP;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int LOADS = BC * CPR / 256; // 16-byte chunks per thread per tile, each of K and V
  static constexpr int ROWS_PER_LOAD = 256 / CPR;
};

}  // namespace

template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_fwd_kernel(
    const char* __restrict__ q, const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ o,
    int batch, int hq, int hkv, int n, float c, int num_q_tiles) {
  using Cfg = PrefillCfg<D>;
  constexpr int KK = D / 16;  // 32x32x16 k-steps over the head dimension
  constexpr int DT = D / 32;  // 32-row output tiles of the head dimension
  constexpr uint32_t ROWB = 2 * D;
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;

  // Work item.  Workgroups are dealt round-robin to the 8 XCDs (blockIdx % 8),
  // each with its own L2; when the (batch, head) count divides by 8, XCD x is
  // given the heads [x·H/8, (x+1)·H/8) so the K/V it streams stay in its L2.
  // Non-causal: an XCD walks its heads one at a time, all query tiles of a
  // head back to back.  Causal: an XCD interleaves its heads and walks query
  // tiles longest-first, which balances the triangular work.
  const int H = batch * hq;
  int bh, qt;
  if (H % 8 == 0) {
    const int per = H / 8;
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    if (CAUSAL) {
      bh = xcd * per + slot % per;
      qt = num_q_tiles - 1 - slot / per;
    } else {
      bh = xcd * per + slot / num_q_tiles;
      qt = slot % num_q_tiles;
    }
  } else {
    bh = blockIdx.x % H;
    qt = CAUSAL ? num_q_tiles - 1 - (int)(blockIdx.x / H) : (int)(blockIdx.x / H);
  }
  const int h = bh % hq;
  const int b = bh / hq;
  const int kvh = h / (hq / hkv);

  const int q0 = qt * Cfg::BR;
  const int qw = q0 + wave * 32;
  const int qrow = qw + (lane & 31);
  const size_t qo_base = ((size_t)b * hq + h) * (size_t)n * ROWB;
  const size_t kv_base = ((size_t)b * hkv + kvh) * (size_t)n * ROWB;
  const char* kp = k + kv_base;
  const char* vp = v + kv_base;

  // Q operand (B of Sᵀ = K·Qᵀ): lane holds query qrow, head-dim elements kk·16 + 8·half .. +7
  u32x4 qf[KK];
  {
    const char* qp = q + qo_base + (size_t)qrow * ROWB;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = qrow < n ? gload16(qp + (kk * 16 + 8 * half) * 2) : zero4();
  }

  const int kend = CAUSAL ? min(n, q0 + Cfg::BR) : n;  // keys any row of this workgroup can see
  const int nkt = (kend + Cfg::BC - 1) / Cfg::BC;
  const int wave_last = min(n - 1, qw + 31);          // last live query row of this wave

  // Tile loads: thread tid moves chunk (tid % CPR) of rows tid/CPR + i·ROWS_PER_LOAD.
  const uint32_t g_off = (uint32_t)(tid / Cfg::CPR) * ROWB + (tid % Cfg::CPR) * 16;
  const uint32_t k_st = (uint32_t)(tid / Cfg::CPR) * Cfg::KP + (tid % Cfg::CPR) * 16;
  const uint32_t v_st = Cfg::KBYTES + (uint32_t)(tid / Cfg::CPR) * Cfg::VP + (tid % Cfg::CPR) * 16;
  u32x4 kst[Cfg::LOADS], vst[Cfg::LOADS];
  auto load_tile = [&](int it) {
    // rows [j0, j0 + BC) of this head, clipped to the sequence: rows past n read as 0
    const int j0 = min(it * Cfg::BC, n);
    const uint32_t bytes = (uint32_t)min(Cfg::BC, n - j0) * ROWB;
    const bufres rk = make_bufres(kp + (size_t)j0 * ROWB, bytes);
    const bufres rv = make_bufres(vp + (size_t)j0 * ROWB, bytes);
#pragma unroll
    for (int i = 0; i < Cfg::LOADS; ++i) {
      kst[i] = bload16(rk, g_off + i * Cfg::ROWS_PER_LOAD * ROWB);
      vst[i] = bload16(rv, g_off + i * Cfg::ROWS_PER_LOAD * ROWB);
    }
  };
  auto store_tile = [&](int stage) {
    char* base = lds + stage * Cfg::STAGE;
#pragma unroll
    for (int i = 0; i < Cfg::LOADS; ++i) {
      lds_write16(base, k_st + i * Cfg::ROWS_PER_LOAD * Cfg::KP, kst[i]);
      lds_write16(base, v_st + i * Cfg::ROWS_PER_LOAD * Cfg::VP, vst[i]);
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;

  // per-lane LDS bases: K operand row, V transpose-read block
  const int G = lane >> 4, j = lane & 15;
  const uint32_t k_rd = (lane & 31) * Cfg::KP + half * 16;
  const uint32_t v_rd = Cfg::KBYTES + (4 * (G >> 1) + (j >> 2)) * Cfg::VP + (16 * (G & 1) + 4 * (j & 3)) * 2;

  auto compute = [&](int stage, int it) {
    const int j0 = it * Cfg::BC;
    if (CAUSAL && j0 > wave_last) return;  // the whole tile lies above this wave's diagonal
    const char* st = lds + stage * Cfg::STAGE;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int s0 = j0 + 32 * sb;
      // Sᵀ subtile: s[e] is key s0 + 8·(e/4) + 4·half + e%4 against query qrow
      f32x16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) s = T::mfma32(lds_read16(st, k_rd + sb * 32 * Cfg::KP + kk * 32), qf[kk], s);

      if (s0 + 32 > n || (CAUSAL && s0 + 31 > qw)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = s0 + 8 * (e >> 2) + 4 * half + (e & 3);
          if (key >= n || (CAUSAL && key > qrow)) s[e] = kNegInf;
        }
      }

      float mx = fmaxf(s[0], s[1]);
#pragma unroll
      for (int e = 2; e < 16; e += 2) mx = fmaxf(mx, fmaxf(s[e], s[e + 1]));
      const float m_tile = max_xor32(mx) * c;  // the subtile's row max, exp2 domain
      // Raise the reference maximum only when some row's new maximum exceeds it
      // by more than kRescaleLog2; then l and o are rescaled by
      // exp2(m_run - m_new) (0 on the first live subtile).  Otherwise every
      // p stays <= 2^kRescaleLog2.  The test is wave-uniform.
      if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleLog2) != 0) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == kNegInf) ? 0.f : m_run;  // a row with no live key yet stays empty
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = fast_exp2(fmaf(s[e], c, -m_use));

      // P, rounded to the storage type, as the B operand of Oᵀ += Vᵀ·Pᵀ (one
      // 16-key k-step per ks); l adds up exactly these rounded weights.
      u32x4 pf[2];
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[ks][i] = T::pack2(s[8 * ks + 2 * i], s[8 * ks + 2 * i + 1]);
          if (i & 1)
            ps1 = T::add_pair(ps1, pf[ks][i]);
          else
            ps0 = T::add_pair(ps0, pf[ks][i]);
        }
      l_run += ps0 + ps1;

      // V operand (A of Oᵀ += Vᵀ·Pᵀ): lane (group G of 16, index j) takes head-dim column
      // 32·dt + 16·(G&1) + j and keys 32·sb + 16·ks + 4·(G>>1) + {0..3} and the same + 8
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint32_t off = v_rd + (32 * sb + 16 * ks) * Cfg::VP + dt * 64;
          const u32x2 va = lds_read_tr16(st, off);
          const u32x2 vb = lds_read_tr16(st, off + 8 * Cfg::VP);
          oacc[dt] = T::mfma32(u32x4{va[0], va[1], vb[0], vb[1]}, pf[ks], oacc[dt]);
        }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  // Unrolled by two so each LDS stage is addressed with immediates.  The next
  // tile is always prefetched: past the last tile the loads read 0 (or
  // in-range rows nobody uses) into a stage that is never read.
  for (int it = 0;;) {
    load_tile(it + 1);
    compute(0, it);
    store_tile(1);
    __syncthreads();
    if (++it >= nkt) break;
    load_tile(it + 1);
    compute(1, it);
    store_tile(0);
    __syncthreads();
    if (++it >= nkt) break;
  }

  // epilogue: O = o / l, rounded to the storage type, written once
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < n) {
    char* op = o + qo_base + (size_t)qrow * ROWB;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int eh = 0; eh < 4; ++eh) {
        const int dcol = dt * 32 + 8 * eh + 4 * half;
        const u32x2 w = {T::pack2(oacc[dt][4 * eh + 0] * inv, oacc[dt][4 * eh + 1] * inv),
                         T::pack2(oacc[dt][4 * eh + 2] * inv, oacc[dt][4 * eh + 3] * inv)};
        gstore8(op + dcol * 2, w);
      }
  }
}

template <class T, int D, bool CAUSAL>
static hipError_t launch_prefill_t(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                                   int n, float scale, hipStream_t stream) {
  using Cfg = PrefillCfg<D>;
  const int tiles = (n + Cfg::BR - 1) / Cfg::BR;
  const long long blocks = (long long)tiles * hq * batch;
  prefill_fwd_kernel<T, D, CAUSAL><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      static_cast<const char*>(q), static_cast<const char*>(k), static_cast<const char*>(v), static_cast<char*>(o),
      batch, hq, hkv, n, scale * kLog2e, tiles);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_prefill_d(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                                   int n, float scale, bool causal, hipStream_t stream) {
  return causal ? launch_prefill_t<T, D, true>(q, k, v, o, batch, hq, hkv, n, scale, stream)
                : launch_prefill_t<T, D, false>(q, k, v, o, batch, hq, hkv, n, scale, stream);
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, void* o, bool bf16, int batch, int hq,
                          int hkv, int n, int d, float scale, bool causal, hipStream_t stream) {
  if (bf16)
    return d == 64 ? launch_prefill_d<Bf16, 64>(q, k, v, o, batch, hq, hkv, n, scale, causal, stream)
                   : launch_prefill_d<Bf16, 128>(q, k, v, o, batch, hq, hkv, n, scale, causal, stream);
  return d == 64 ? launch_prefill_d<F16, 64>(q, k, v, o, batch, hq, hkv, n, scale, causal, stream)
                 : launch_prefill_d<F16, 128>(q, k, v, o, batch, hq, hkv, n, scale, causal, stream);
}

}  // namespace attn
