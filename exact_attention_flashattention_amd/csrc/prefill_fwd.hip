// Prefill forward: exact attention of a square problem, tile by tile.
//
// FlashAttention as described in "FlashAttention: what never touches memory"
// ("Attention from the kernel's side") and "03 · The structure" ("Quantized
// kernels"): a block of query rows stays resident, tiles of K and V stream
// past it through on-chip memory, each tile's scores update the running
// (m, l, o) of every row with the online-softmax recurrence, and O is written
// once.  Scores and probabilities exist only in registers.
//
// gfx950 mapping.  One workgroup = 4 wavefronts = 256 query rows; each wave
// owns 64 rows as two 32-row blocks, so every K or V fragment read from LDS
// feeds two matrix instructions (LDS read bandwidth, not the matrix cores,
// limits a 32-row-per-wave design on this chip).
//   * Q rows sit in registers as the B operand of 32x32x16 MFMA.
//   * K and V tiles of 64 keys go from HBM/L2 straight into LDS with
//     buffer-load-to-LDS (no register staging; rows past the sequence end
//     read as 0).  Three LDS stages: the tile being consumed, the tile whose
//     last P·V is still in flight, and the tile being fetched -- one barrier
//     per tile.  Rows are stored unpadded with an XOR swizzle of their 16-byte
//     chunks, chosen so the K operand reads (ds_read_b128) and the V
//     transpose reads (ds_read_b64_tr_b16) are free of bank conflicts.
//   * Scores are computed transposed, Sᵀ = K·Qᵀ, so each lane holds keys of
//     ONE query: the row max is an in-lane max plus one exchange between the
//     wave's halves (v_permlane32_swap), and the rescale factor is one scalar
//     per lane.  K rows enter the MFMA in an order that swaps bits 2 and 3 of
//     the row index, which leaves every lane's probabilities for each 16-key
//     k-step on 8 consecutive keys -- exactly the B operand of
//     Oᵀ += Vᵀ·Pᵀ, with no shuffle.
//   * V reaches the matrix cores through the LDS transpose read, which hands
//     each lane 4 consecutive keys of one head-dimension column.
//   * Software pipelining in program order, per 32-key subtile:
//     exponentials of this subtile, score MFMAs of the next, P·V MFMAs of
//     this one, row max of the next -- neighbouring matrix and vector work is
//     independent, so the two units overlap within a wave.
//   * The softmax runs in the exp2 domain (scale·log2 e folded into one FMA
//     per score, v_exp_f32).  The reference maximum is raised only when a
//     row's new maximum exceeds it by more than 2^8; o and l share the
//     reference, so o/l is unchanged and the output rescale stays off the
//     common path.
//   * Causal: key tiles wholly above a wave's diagonal cost that wave
//     nothing, the mask is applied only on subtiles that cross the diagonal
//     or the sequence end (block classification of "Masking variants",
//     "Attention Computation in Practice" section 5), and the longest query
//     tiles are launched first.
#include "device_common.hpp"
#include "launchers.hpp"

namespace attn {

namespace {

// Largest growth of a row maximum (in log2 units) absorbed without rescaling.
constexpr float kRescaleLog2 = 8.f;

// Per head dimension: NB 32-row query blocks per wave and the number of LDS
// stages.  d=64 takes two blocks (64 rows per wave) and three stages; at d=128
// two blocks' output accumulators and Q operands alone would fill the register
// budget of two waves per SIMD, so it takes one block and two stages.  Both run
// two waves per SIMD, so one wave's softmax also overlaps the other's MFMAs.
template <int D>
struct PrefillCfg {
  static constexpr int NB = D == 64 ? 2 : 1;
  static constexpr int WAVES = 4;
  static constexpr int BR = 32 * NB * WAVES;    // query rows per workgroup
  static constexpr int BC = 64;                 // keys per tile (two 32-key subtiles)
  static constexpr int ROWB = 2 * D;            // bytes per K/V row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int TILE = BC * ROWB;        // bytes of one K (or V) tile
  static constexpr int STAGE = 2 * TILE;        // K tile then V tile
  static constexpr int STAGES = D == 64 ? 3 : 2;
  static constexpr int LDS = STAGES * STAGE;
  static constexpr int DMA = TILE / 16 / 256;   // 1 KB wave transfers per thread per tensor per tile
  static constexpr int WAVES_PER_EU = 2;
};

// Chunk swizzles (physical 16-byte chunk = logical chunk ^ swizzle(row)).
// K: a wave reads 32 rows at one logical chunk; every 16 of them must land on
// distinct bank groups.  V: each 16-lane group reads 4 rows x 2 adjacent
// chunks; those 8 must land on distinct bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? ((r & 7) << 1) : (r & 6);
}

// MFMA row i of a 32-key subtile carries key perm_row(i): bits 2 and 3 swapped.
__device__ __forceinline__ int perm_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

}  // namespace

template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PrefillCfg<D>::WAVES_PER_EU,
                                                                     PrefillCfg<D>::WAVES_PER_EU))) void
prefill_fwd_kernel(const char* __restrict__ q, const char* __restrict__ k, const char* __restrict__ v,
                   char* __restrict__ o, int batch, int hq, int hkv, int n, float c, int num_q_tiles) {
  using Cfg = PrefillCfg<D>;
  constexpr int NB = Cfg::NB;
  constexpr int KK = D / 16;  // 32x32x16 k-steps over the head dimension
  constexpr int DT = D / 32;  // 32-row output tiles of the head dimension
  constexpr uint32_t ROWB = Cfg::ROWB;
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep it (and
  // the LDS-DMA destinations and buffer resources derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

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
  const int qw = q0 + wave * 32 * NB;  // first query row of this wave; block blk covers qw + 32·blk ..
  const size_t qo_base = ((size_t)b * hq + h) * (size_t)n * ROWB;
  const size_t kv_base = ((size_t)b * hkv + kvh) * (size_t)n * ROWB;
  const char* kp = k + kv_base;
  const char* vp = v + kv_base;

  // Q operands (B of Sᵀ = K·Qᵀ): block blk, lane holds query qw + 32·blk + l32,
  // head-dim elements 16·kk + 8·half .. +7
  u32x4 qf[NB][KK];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int qrow = qw + 32 * blk + l32;
    const char* qp = q + qo_base + (size_t)qrow * ROWB;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[blk][kk] = qrow < n ? gload16(qp + (kk * 16 + 8 * half) * 2) : zero4();
  }

  const int kend = CAUSAL ? min(n, q0 + Cfg::BR) : n;  // keys any row of this workgroup can see
  const int nkt = (kend + Cfg::BC - 1) / Cfg::BC;
  const int wave_last = min(n - 1, qw + 32 * NB - 1); // last live query row of this wave

  // ---- tile fetch: 1 KB wave transfers straight into LDS.  Transfer g = i·WAVES + wave
  // fills bytes [g·1024, g·1024 + 1024) of the tile; lane l fills slot g·64 + l, i.e.
  // physical chunk (slot % CPR) of row slot / CPR, with the logical chunk that maps there.
  // Row / CPR arithmetic makes the swizzle of every transfer of a lane the same.
  const int slot_row = (wave * 64 + lane) / Cfg::CPR;
  const int slot_chunk = lane % Cfg::CPR;
  const uint32_t k_src = slot_row * ROWB + ((slot_chunk ^ swz_k<D>(slot_row)) * 16);
  const uint32_t v_src = slot_row * ROWB + ((slot_chunk ^ swz_v<D>(slot_row)) * 16);
  auto fetch_tile = [&](int it, int stage) {
    const int j0 = min(it * Cfg::BC, n);
    const int bytes = min(Cfg::BC, n - j0) * (int)ROWB;  // rows past the end read as 0
    const char* kt = kp + (size_t)j0 * ROWB;
    const char* vt = vp + (size_t)j0 * ROWB;
    const uint32_t st = lds_addr(lds) + stage * Cfg::STAGE;
#pragma unroll
    for (int i = 0; i < Cfg::DMA; ++i) {
      const int first = i * Cfg::WAVES * 1024;          // the transfer group's first byte in the tile
      const uint32_t off = first + wave * 1024;         // this wave's transfer
      const int rec = bytes > first ? bytes - first : 0;
      dma16_to_lds(bufres_words(kt + first, (uint32_t)rec), k_src, st + off);
      dma16_to_lds(bufres_words(vt + first, (uint32_t)rec), v_src, st + Cfg::TILE + off);
    }
  };

  // ---- per-lane LDS read offsets (within a stage)
  // K operand of k-step kk: row perm_row(l32) of the subtile, logical chunk 2·kk + half
  uint32_t k_rd[KK];
  {
    const int r = perm_row(l32);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) k_rd[kk] = r * ROWB + (((2 * kk + half) ^ swz_k<D>(r)) * 16);
  }
  // V operand of output tile dt: 16-lane group G, index j reads rows
  // 16·ks + 8·(G>>1) + j/4 (+4 for the second read) at head-dim columns
  // 32·dt + 16·(G&1) + 4·(j&3) .. +3
  uint32_t v_rd[DT][2];
  {
    const int G = lane >> 4, j = lane & 15;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 8 * (G >> 1) + (j >> 2) + 4 * p;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int lc = dt * 4 + 2 * (G & 1) + ((j & 3) >> 1);
        v_rd[dt][p] = Cfg::TILE + r * ROWB + ((lc ^ swz_v<D>(r)) * 16) + 8 * (j & 1);
      }
    }
  }

  float m_run[NB], l_run[NB];
  f32x16 oacc[NB][DT];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    m_run[blk] = kNegInf;
    l_run[blk] = 0.f;
  }
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[blk][dt][e] = 0.f;

  // scores of subtile sb of the tile in `stage`: s[blk][e] is key
  // 16·(e>>3) + 8·half + (e&7) of the subtile against query qw + 32·blk + l32
  auto qk = [&](f32x16 (&s)[NB], int stage, int sb) {
    const char* st = lds + stage * Cfg::STAGE + sb * 32 * ROWB;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[blk][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 kf = lds_read16(st, k_rd[kk]);
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) s[blk] = T::mfma32(kf, qf[blk][kk], s[blk]);
    }
  };

  // mask, row max and (rarely) the rescale of one subtile's scores starting at key s0
  auto row_max = [&](f32x16 (&s)[NB], int s0) {
    if (s0 + 32 > n || (CAUSAL && s0 + 31 > qw)) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int qrow = qw + 32 * blk + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = s0 + 16 * (e >> 3) + 8 * half + (e & 7);
          if (key >= n || (CAUSAL && key > qrow)) s[blk][e] = kNegInf;
        }
      }
    }
    float m_tile[NB];
    bool grow = false;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      float mx = fmaxf(s[blk][0], s[blk][1]);
#pragma unroll
      for (int e = 2; e < 16; e += 2) mx = fmaxf(mx, fmaxf(s[blk][e], s[blk][e + 1]));
      m_tile[blk] = max_xor32(mx) * c;
      grow |= m_tile[blk] > m_run[blk] + kRescaleLog2;
    }
    // Raise the reference maximum only when some row's new maximum exceeds it
    // by more than kRescaleLog2 (always on a row's first live subtile); l and o
    // are rescaled by exp2(m_run - m_new), which is 0 while m_run = -inf.
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const float m_new = fmaxf(m_run[blk], m_tile[blk]);
        const float alpha = fast_exp2(m_run[blk] - (m_new == kNegInf ? 0.f : m_new));
        l_run[blk] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[blk][dt] *= alpha;
        m_run[blk] = m_new;
      }
    }
  };

  // probabilities rounded to the storage type as the B operands of P·V (one per
  // 16-key k-step), and their row sums
  auto exp_pack = [&](f32x16 (&s)[NB], u32x4 (&pf)[NB][2]) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const float m_use = (m_run[blk] == kNegInf) ? 0.f : m_run[blk];  // a row with no live key stays empty
#pragma unroll
      for (int e = 0; e < 16; ++e) s[blk][e] = fast_exp2(fmaf(s[blk][e], c, -m_use));
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[blk][ks][i] = T::pack2(s[blk][8 * ks + 2 * i], s[blk][8 * ks + 2 * i + 1]);
          if (i & 1)
            ps1 = T::add_pair(ps1, pf[blk][ks][i]);
          else
            ps0 = T::add_pair(ps0, pf[blk][ks][i]);
        }
      l_run[blk] += ps0 + ps1;
    }
  };

  auto pv = [&](const u32x4 (&pf)[NB][2], int stage, int sb) {
    const char* st = lds + stage * Cfg::STAGE + sb * 32 * ROWB;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x2 va = lds_read_tr16(st + ks * 16 * ROWB, v_rd[dt][0]);
        const u32x2 vb = lds_read_tr16(st + ks * 16 * ROWB, v_rd[dt][1]);
        const u32x4 vf = {va[0], va[1], vb[0], vb[1]};
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) oacc[blk][dt] = T::mfma32(vf, pf[blk][ks], oacc[blk][dt]);
      }
  };

  // ---- pipeline.  Invariant at the top of a tile step: the tile is in LDS and
  // visible, the next tile is in flight, and `s` holds the (masked, max-applied)
  // scores of this tile's subtile 0.
  f32x16 s[NB], s_next[NB];
  u32x4 pf[NB][2];

  fetch_tile(0, 0);
  wait_vm_all();
  __syncthreads();
  if (nkt > 1) fetch_tile(1, 1);
  bool live = !CAUSAL || 0 <= wave_last;
  if (live) {
    qk(s, 0, 0);
    row_max(s, 0);
  }

  auto tile_step = [&](int it, int stage) {
    const int j0 = it * Cfg::BC;
    const bool live0 = !CAUSAL || j0 <= wave_last;
    const bool live1 = !CAUSAL || j0 + 32 <= wave_last;
    // subtile 0: exponentials, next subtile's scores, this subtile's P·V
    if (live0) {
      exp_pack(s, pf);
      if (live1) qk(s_next, stage, 1);
      pv(pf, stage, 0);
      if (live1) row_max(s_next, j0 + 32);
    }
    // subtile 1 and the hand-over to the next tile.  With three stages the
    // next tile's first scores are issued before this subtile's P·V (its stage
    // is not refilled until the next barrier); with two, this tile's stage is
    // refilled right after the barrier, so its P·V must come first.
    const int nstage = (stage + 1) % Cfg::STAGES;
    const bool more = it + 1 < nkt;
    const bool live2 = more && (!CAUSAL || j0 + 64 <= wave_last);
    if (live1) exp_pack(s_next, pf);
    if (Cfg::STAGES == 2 && live1) pv(pf, stage, 1);
    if (more) {
      wait_vm_all();   // the next tile has landed (this wave's part)
      __syncthreads(); // ... everyone's part; every wave is past its last read of the stage refilled next
      if (it + 2 < nkt) fetch_tile(it + 2, (stage + 2) % Cfg::STAGES);
      if (live2) qk(s, nstage, 0);
    }
    if (Cfg::STAGES == 3 && live1) pv(pf, stage, 1);
    if (live2) row_max(s, j0 + 64);
  };

  // unrolled by the stage count so each stage is a compile-time constant
  for (int it = 0;;) {
    tile_step(it, 0);
    if (++it >= nkt) break;
    tile_step(it, 1);
    if (++it >= nkt) break;
    if (Cfg::STAGES == 3) {
      tile_step(it, 2);
      if (++it >= nkt) break;
    }
  }

  // ---- epilogue: O = o / l, rounded to the storage type, written once
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const float l_tot = sum_xor32(l_run[blk]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int qrow = qw + 32 * blk + l32;
    if (qrow < n) {
      char* op = o + qo_base + (size_t)qrow * ROWB;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int eh = 0; eh < 4; ++eh) {
          const int dcol = dt * 32 + 8 * eh + 4 * half;
          const u32x2 w = {T::pack2(oacc[blk][dt][4 * eh + 0] * inv, oacc[blk][dt][4 * eh + 1] * inv),
                           T::pack2(oacc[blk][dt][4 * eh + 2] * inv, oacc[blk][dt][4 * eh + 3] * inv)};
          gstore8(op + dcol * 2, w);
        }
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
