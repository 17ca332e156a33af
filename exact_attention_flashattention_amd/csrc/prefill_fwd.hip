// Prefill forward: exact attention of a square problem, tile by tile.
//
// FlashAttention as described in "FlashAttention: what never touches memory"
// ("Attention from the kernel's side") and "03 · The structure" ("Quantized
// kernels"): a block of query rows stays resident, tiles of K and V stream
// past it through on-chip memory, each tile's scores update the running
// (m, l, o) of every row with the online-softmax recurrence, and O is written
// once.  Scores and probabilities exist only in registers.
//
// gfx950 mapping.  One workgroup = 8 wavefronts, two per SIMD, each owning NB
// blocks of 32 query rows (two at d=64, one at d=128); the K/V tiles in LDS
// are shared by all eight.
//   * Two wave groups run anti-phased.  Every wave alternates a matrix step
//     (score MFMAs of one 32-key subtile, P·V MFMAs of the previous one, and
//     between them the LDS reads of the K and V operands of the next matrix
//     step) and a vector step (mask, exponentials, packing and the raise test
//     of a subtile, and the tile transfers; the rare raise itself -- row max
//     and rescale -- runs after the step's barrier).  Group 1 runs one step
//     behind group 0
//     and every step ends at a workgroup barrier, so on each SIMD one wave
//     keeps the matrix core busy while its partner does the softmax
//     arithmetic -- the two units overlap instead of taking turns.  The
//     vector step is the longer of the two, so it carries no operand reads.
//   * Q rows sit in registers as the B operand of 32x32x16 MFMA.
//   * K and V tiles of 64 keys go from HBM/L2 straight into LDS with
//     buffer-load-to-LDS (rows past the sequence end read as 0), into one of
//     STAGES buffers; a tile is fetched as soon as both groups are done with
//     the tile that last used its buffer, and each wave waits for its own
//     part with an exact vmcnt before the barrier that precedes the tile's
//     first read.  Rows are stored unpadded with an XOR swizzle of their
//     16-byte chunks so the K operand reads (ds_read_b128) and the V
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
//   * The softmax runs in the exp2 domain (scale·log2 e folded into one FMA
//     per score, v_exp_f32).  The reference maximum is raised only when a
//     row's probabilities grow past 2^8; o and l share the reference, so o/l
//     is unchanged and the output rescale stays off the common path.  At d=64
//     the row sums l run on the matrix cores (one small MFMA per 16 keys), at
//     d=128 on the vector unit (v_dot2 over the packed probabilities).
//   * Causal: subtiles wholly above a wave's diagonal cost that wave nothing,
//     the mask is applied only on subtiles that cross the diagonal or the
//     sequence end (block classification of "Masking variants", "Attention
//     Computation in Practice" section 5), and the longest query tiles are
//     launched first.
//
// Variable-length batches (VARLEN = true; the append / mixed kernel of "The
// four attention kernels you actually use", same section): sequences are
// packed token-major, Q and O [total_q, hq, d], K and V [total_k, hkv, d], and
// sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows
// cu_k[b] .. cu_k[b+1]-1.  Its nq queries are the LAST nq of its nk positions
// (bottom-right alignment), so under the causal mask query i sees keys
// j <= i + nk - nq; a square problem is the case nq = nk.  The only changes
// are the row strides (a runtime value instead of the row size), the
// per-sequence bases and lengths, and workgroups past a sequence's last query
// tile returning at once.
//
// Masking variants of the same section, both run-time options: a sliding
// window W keeps key j for the query at position p iff p - W < j <= p (the
// workgroup starts at the first key tile its first row's window reaches, so
// the window skips tiles on the left as the diagonal skips them on the
// right); ALiBi adds -m_h·(p - j) to every score of query head h (slopes m_h
// given per query head), folded into the raw scores as (m_h / scale)·(j - p)
// before the exponentials.
#include "device_common.hpp"
#include "launchers.hpp"

#include <atomic>
#include <type_traits>

namespace attn {

namespace {

// NB 32-row query blocks per wave: two at d=64; one at d=128, where two
// blocks' accumulators and Q operands would not fit two waves per SIMD.
template <int D>
struct PrefillCfg {
  static constexpr int NB = D == 64 ? 2 : 1;
  static constexpr int WAVES = 8;               // two groups of four, two waves per SIMD
  static constexpr int BR = 32 * NB * WAVES;    // query rows per workgroup
  static constexpr int BC = 64;                 // keys per tile (two 32-key subtiles)
  static constexpr int ROWB = 2 * D;            // bytes per K/V row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int TILE = BC * ROWB;        // bytes of one K (or V) tile
  static constexpr int STAGES = 4;              // LDS tile buffers
  static constexpr int VREG = STAGES * TILE;    // K tiles of all buffers first, then the V tiles
  static constexpr int LDS = 2 * VREG;
  static constexpr int DMA = TILE / 16 / (64 * WAVES);  // 1 KB transfers per wave per tensor per tile
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

// s_waitcnt vmcnt(N), other counters untouched (gfx9 field layout).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// End of a step: a workgroup barrier that nothing is scheduled across.  No
// memory fence: buffer-to-LDS loads in flight stay in flight, their
// completion is awaited explicitly.  A vector step (at d=64 only the second of
// a tile, and the set-up and final steps) also waits for this wave's LDS
// reads, so that once the barrier opens nothing this wave read can still be
// pending when a later tile fetch overwrites it; the other steps leave their
// reads in flight and go straight to the barrier (a tile's buffer is refilled
// only after both groups have passed a second vector step since its last
// read, see the fetch schedule below).
template <bool WAIT_LDS>
__device__ __forceinline__ void step_end() {
  __builtin_amdgcn_sched_barrier(0);  // keep the wait below the step's own work
  if (WAIT_LDS) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// A wave-uniform pointer placed in scalar registers (the compiler may have
// computed it with vector instructions, e.g. through an integer division).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// f(integral_constant<int, i>) for i = I .. N-1, each index a compile-time value.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Kernel-local helpers are lambdas; all of them are inlined (a call would
// spill the operand registers to scratch memory).
#define ATTN_INLINE __attribute__((always_inline))

// Pins a value in registers at this point of the program: the empty asm
// statement reads and rewrites it, so whatever computes the value stays before
// it and whatever uses the result stays after.  Used at the end of each step,
// so the compiler cannot move one step's arithmetic into the next one.
template <class V>
__device__ __forceinline__ void pin(V& x) {
  asm volatile("" : "+v"(x));
}

}  // namespace

// Sequence bounds of a variable-length batch (unused by the square kernel).
struct VarlenArgs {
  const int* cu_q;  // [batch + 1] query row offsets
  const int* cu_k;  // [batch + 1] key row offsets
  int total_q;      // rows of Q / O; every sequence is clamped into [0, total_q)
  int total_k;      // rows of K / V; likewise
  int max_k;        // most keys per sequence
};

// Masking variants (zero / null: none).
struct MaskArgs {
  int window;          // > 0: sliding window of this many keys (causal kernels only)
  const float* alibi;  // [hq] ALiBi slopes, natural-log units per position
};

// One work item (a query tile of one head, see below) of a workgroup: item
// `bid`.  `qf` holds the Q operands; with have_q they were read already (by
// the previous item's prefetch).  next_bid >= 0 (square non-causal kernels
// only): the workgroup's next item, whose Q operands are read into `qf` once
// this item's last score MFMA has used them.
template <class T, int D, bool CAUSAL, bool VARLEN>
__device__ __forceinline__ void prefill_item(
    const int bid, const int next_bid, u32x4 (&qf)[PrefillCfg<D>::NB][D / 16], const bool have_q,
    const char* __restrict__ q, const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ o,
    int batch, int hq, int hkv, int n, float c, int num_q_tiles, VarlenArgs vl, MaskArgs mk) {
  using Cfg = PrefillCfg<D>;
  constexpr int NB = Cfg::NB;
  constexpr int KK = D / 16;  // 32x32x16 k-steps over the head dimension
  constexpr int DT = D / 32;  // 32-row output tiles of the head dimension
  constexpr int S = Cfg::STAGES;
  constexpr uint32_t ROWB = Cfg::ROWB;
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS];

  // The thread index passes through an opaque move, so that nothing derived
  // from it is hoisted out of the work-item loop of the persistent kernels
  // (kept live across the loop, that set-up spills).
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  const int lane = tid & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep it (and
  // the LDS-DMA destinations and buffer resources derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // waves w and w+4 share a SIMD and sit in different groups
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Work item.  Workgroups are dealt round-robin to the 8 XCDs (blockIdx % 8,
  // which equals bid % 8 since a persistent grid is a multiple of 8), each
  // with its own L2; when the (batch, head) count divides by 8, XCD x is
  // given the heads [x·H/8, (x+1)·H/8) so the K/V it streams stay in its L2.
  // Non-causal: an XCD walks its heads one at a time, all query tiles of a
  // head back to back.  Causal: an XCD interleaves its heads and walks query
  // tiles longest-first, which balances the triangular work.
  // Variable-length batches: (sequence, KV head) units are dealt round-robin
  // to the XCDs instead, so that with hkv a multiple of 8 every XCD holds the
  // same KV heads of every sequence -- unequal sequences then load all XCDs
  // alike -- and the query heads sharing a KV head stay on one XCD.  An XCD
  // takes its units one after another, each unit's query tiles from the last
  // down with the unit's query heads side by side, so the tiles that stream
  // the same K and V run close together and share them in the XCD's L2.  The
  // units go in order of key count, most first, so that the XCD's share ends
  // on the shortest work items; their work items are numbered back to back,
  // and the workgroups past the last one (the grid is sized for every unit
  // having the longest sequence's tiles) come last and exit at once.  (With
  // more than 64 units per XCD the units keep their index order, each given
  // that many workgroups.)
  // A sequence's last query tile is usually partial; its rows fill only the
  // first nb of the 8 waves' row blocks, and since the query heads of a unit
  // see the same keys under the same mask, one workgroup takes that tile for
  // P = min(g, 8 / nb) of them: wave w serves head w / nb, row block w % nb
  // (waves left over hold no rows).  The unit's other tiles are whole.
  int b, h, qt;
  int wrow = wave;   // this wave's row block within the query tile
  bool live = true;  // false: a wave of a shared last tile with no head to serve
  int nq = n, nk = n;
  size_t qo_base, kv_base;
  const uint32_t q_stride = VARLEN ? (uint32_t)hq * ROWB : ROWB;
  const uint32_t kv_stride = VARLEN ? (uint32_t)hkv * ROWB : ROWB;
  if constexpr (VARLEN) {
    const int g = hq / hkv;
    const int xcd = bid % 8, slot = bid / 8;
    const int units = (batch * hkv - xcd + 7) / 8;  // units of this XCD: xcd, xcd + 8, ...
    // row bounds of sequence bb, clamped into the buffers
    auto bounds = [&](int bb, int& qs_, int& qe_, int& ks_, int& ke_) ATTN_INLINE {
      qs_ = min(max(vl.cu_q[bb], 0), vl.total_q);
      qe_ = min(max(vl.cu_q[bb + 1], qs_), min(vl.total_q, qs_ + n));
      ks_ = min(max(vl.cu_k[bb], 0), vl.total_k);
      ke_ = min(max(vl.cu_k[bb + 1], ks_), min(vl.total_k, ks_ + vl.max_k));
    };
    // query tiles of nq_ rows; row blocks of the last one, query heads per
    // workgroup on it, and its workgroups
    auto tiling = [&](int nq_, int& tiles_, int& nb_, int& P_, int& np_) ATTN_INLINE {
      tiles_ = (nq_ + Cfg::BR - 1) / Cfg::BR;
      nb_ = max(1, (nq_ - (tiles_ - 1) * Cfg::BR + 32 * NB - 1) / (32 * NB));
      P_ = min(g, Cfg::WAVES / nb_);
      np_ = (g + P_ - 1) / P_;
    };
    int unit, j, qs, qe, ks, ke;
    if (units <= 64) {
      // lane l describes unit xcd + 8l: its bounds, key count and work items
      int lqs = 0, lqe = 0, lks = 0, lke = 0, lnk = -1, items = 0;
      if (lane < units) {
        bounds((xcd + 8 * lane) / hkv, lqs, lqe, lks, lke);
        int tl, nbl, Pl, npl;
        tiling(lqe - lqs, tl, nbl, Pl, npl);
        items = tl == 0 ? 0 : npl + (tl - 1) * g;
        lnk = lke - lks;
      }
      // the work items of the units ahead of lane l's (more keys, or as many and a lower index)
      int start = 0;
      for (int u = 0; u < units; ++u) {
        const int ku = __builtin_amdgcn_readlane(lnk, u);
        const int iu = __builtin_amdgcn_readlane(items, u);
        start += (ku > lnk || (ku == lnk && u < lane)) ? iu : 0;
      }
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < units && slot >= start && slot < start + items);
      if (hit == 0) return;  // past this XCD's work items (the whole workgroup)
      const int L = (int)__builtin_ctzll(hit);
      unit = xcd + 8 * L;
      j = slot - __builtin_amdgcn_readlane(start, L);
      qs = __builtin_amdgcn_readlane(lqs, L);
      qe = __builtin_amdgcn_readlane(lqe, L);
      ks = __builtin_amdgcn_readlane(lks, L);
      ke = __builtin_amdgcn_readlane(lke, L);
    } else {
      const int per_unit = g * num_q_tiles;  // workgroups set aside per unit
      if (slot >= units * per_unit) return;  // (the whole workgroup)
      unit = xcd + 8 * (slot / per_unit);
      j = slot % per_unit;
      bounds(unit / hkv, qs, qe, ks, ke);
    }
    b = unit / hkv;
    nq = __builtin_amdgcn_readfirstlane(qe - qs);
    nk = __builtin_amdgcn_readfirstlane(ke - ks);
    int tiles, nb, P, np;
    tiling(nq, tiles, nb, P, np);
    if (tiles == 0) return;
    int head;
    if (j < np) {
      qt = tiles - 1;
      wrow = wave % nb;
      head = j * P + wave / nb;
      live = wave / nb < P && head < g;
      if (!live) head = j * P;
    } else {
      qt = tiles - 2 - (j - np) / g;
      if (qt < 0) return;  // this unit has fewer tiles than the longest sequence (the whole workgroup)
      head = (j - np) % g;
    }
    h = (unit % hkv) * g + head;
    qo_base = ((size_t)qs * hq + h) * ROWB;
    kv_base = ((size_t)ks * hkv + unit % hkv) * ROWB;
  } else {
    const int H = batch * hq;
    int bh;
    if (H % 8 == 0) {
      const int per = H / 8;
      const int xcd = bid % 8, slot = bid / 8;
      if (CAUSAL) {
        bh = xcd * per + slot % per;
        qt = num_q_tiles - 1 - slot / per;
      } else {
        bh = xcd * per + slot / num_q_tiles;
        qt = slot % num_q_tiles;
      }
    } else {
      bh = bid % H;
      qt = CAUSAL ? num_q_tiles - 1 - (int)(bid / H) : (int)(bid / H);
    }
    h = bh % hq;
    b = bh / hq;
    qo_base = ((size_t)b * hq + h) * (size_t)n * ROWB;
    kv_base = ((size_t)b * hkv + h / (hq / hkv)) * (size_t)n * ROWB;
  }
  // Query tile qt of this (sequence, head); the causal diagonal is shifted by
  // off = nk - nq.  A wave with no rows starts at nq, past the last row.
  const int q0 = qt * Cfg::BR;
  const int qw = live ? q0 + wrow * 32 * NB : nq;  // first query row of this wave; block blk covers qw + 32·blk ..
  const int off = VARLEN ? nk - nq : 0;
  const char* kp = k + kv_base;
  const char* vp = v + kv_base;

  // Q operands (B of Sᵀ = K·Qᵀ): block blk, lane holds query qw + 32·blk + l32,
  // head-dim elements 16·kk + 8·half .. +7
  if (!have_q) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int qrow = qw + 32 * blk + l32;
      const char* qp = q + qo_base + (size_t)qrow * q_stride;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[blk][kk] = qrow < nq ? gload16(qp + (kk * 16 + 8 * half) * 2) : zero4();
    }
  }
  // Q operands of the workgroup's next item (square non-causal kernels, heads
  // grouped per XCD as above): read during this item's last vector steps, they
  // arrive while the item finishes and its output is written.
  auto prefetch_q = [&]() ATTN_INLINE {
    const int per = batch * hq / 8;
    const int slot = next_bid / 8;
    const int bh2 = (next_bid % 8) * per + slot / num_q_tiles;
    const int qw2 = (slot % num_q_tiles) * Cfg::BR + wave * 32 * NB;
    const char* q2 = q + (size_t)bh2 * (size_t)n * ROWB;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int qrow = qw2 + 32 * blk + l32;
      const char* qp = q2 + (size_t)qrow * ROWB;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[blk][kk] = qrow < n ? gload16(qp + (kk * 16 + 8 * half) * 2) : zero4();
    }
  };

  // keys any row of this workgroup can see: [key0, kend), key0 a tile boundary
  const int kend = CAUSAL ? max(0, min(nk, q0 + Cfg::BR + off)) : nk;
  const int window = (CAUSAL && VARLEN) ? mk.window : 0;  // the options come with the varlen entry point
  const int key0 = window > 0 ? max(0, q0 + off - window + 1) / Cfg::BC * Cfg::BC : 0;
  const int nkt = VARLEN ? max(0, (kend + Cfg::BC - 1) / Cfg::BC - key0 / Cfg::BC)  // tiles to process
                         : (kend + Cfg::BC - 1) / Cfg::BC;
  // ALiBi slope of this wave's head in raw-score units (the scores are scaled by c = scale·log2 e later)
  const bool alibi = VARLEN && mk.alibi != nullptr;
  const float alibi_raw = alibi ? mk.alibi[h] * kLog2e / c : 0.f;
  if (VARLEN && nkt == 0) {  // no row of this workgroup sees a key: its rows are 0
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int qrow = qw + 32 * blk + l32;
      if (qrow < nq) {
        char* op = o + qo_base + (size_t)qrow * q_stride;
#pragma unroll
        for (int ch = half; ch < Cfg::CPR; ch += 2) gstore16(op + ch * 16, zero4());
      }
    }
    return;
  }

  // ---- tile fetch: 1 KB wave transfers straight into LDS.  Transfer g = i·WAVES + wave
  // fills bytes [g·1024, g·1024 + 1024) of the tile; lane l fills slot g·64 + l, i.e.
  // physical chunk (slot % CPR) of row slot / CPR, with the logical chunk that maps there.
  // Transfer groups start on multiples of 32 rows, so a lane's swizzle is the same in all.
  const int slot_row = (wave * 64 + lane) / Cfg::CPR;
  const int slot_chunk = lane % Cfg::CPR;
  const uint32_t k_src = slot_row * kv_stride + ((slot_chunk ^ swz_k<D>(slot_row)) * 16);
  const uint32_t v_src = slot_row * kv_stride + ((slot_chunk ^ swz_v<D>(slot_row)) * 16);
  constexpr int GROUP_ROWS = Cfg::WAVES * 1024 / ROWB;  // rows of one transfer group
  constexpr int PT = 2 * Cfg::DMA;  // transfers per tile per wave: part j is tensor j&1 (K, V), group j>>1
  // Fetch cursor: scalar state of the next tile to fetch, advanced one tile at a
  // time.  The buffer resources of the tile's transfer groups (each from the
  // group's first row to the sequence end, so rows past the end read as 0) are
  // built when the cursor advances, so issuing a transfer costs an M0 write and
  // the load itself.  (The values are moved to scalar registers explicitly;
  // left to the compiler, parts of them live in vector registers and every
  // transfer pays for the moves.)
  int issued = 0;                                       // transfers this wave has issued so far
  const char* f_k = uniform_ptr(kp + (size_t)key0 * kv_stride);  // K row j0 of the cursor's tile
  const char* f_v = uniform_ptr(vp + (size_t)key0 * kv_stride);  // V row j0
  uint32_t f_rem = (uint32_t)__builtin_amdgcn_readfirstlane(     // bytes from row j0 to the sequence end
      (int)((uint32_t)(nk - key0) * kv_stride));
  i32x4 f_res[2][Cfg::DMA];  // [K, V][transfer group]
  auto make_res = [&]() ATTN_INLINE {
#pragma unroll
    for (int g = 0; g < Cfg::DMA; ++g) {
      const uint32_t src = g * GROUP_ROWS * kv_stride;  // the group's first byte in memory
      const uint32_t rec = f_rem > src ? f_rem - src : 0u;
      f_res[0][g] = bufres_words(f_k + src, rec);
      f_res[1][g] = bufres_words(f_v + src, rec);
    }
  };
  make_res();
  const uint32_t f_dst0 = lds_addr(lds) + wave * 1024;  // this wave's transfers land at stage + g·1024
  uint32_t f_dst = f_dst0;                              // ... of the cursor's stage
  auto fetch_part = [&](auto j_tag) ATTN_INLINE {       // transfer j of the cursor's tile
    constexpr int j = decltype(j_tag)::value;
    // destination: the transfer group's first byte in the tile, in the tensor's region
    dma16_to_lds<(j & 1) * Cfg::VREG + (j >> 1) * Cfg::WAVES * 1024>(f_res[j & 1][j >> 1], (j & 1) ? v_src : k_src,
                                                                     f_dst);
    ++issued;
  };
  auto fetch_advance = [&]() ATTN_INLINE {
    const uint32_t step = Cfg::BC * kv_stride;
    f_k += step;
    f_v += step;
    f_rem = (uint32_t)__builtin_amdgcn_readfirstlane((int)(f_rem > step ? f_rem - step : 0u));
    make_res();
    f_dst = f_dst + Cfg::TILE == f_dst0 + S * Cfg::TILE ? f_dst0 : f_dst + Cfg::TILE;
  };
  auto fetch_tile = [&]() ATTN_INLINE {
    static_for<0, PT>(fetch_part);
    fetch_advance();
  };
  // Wait until every transfer of tiles 0 .. t issued by this wave has landed:
  // vector-memory operations complete in issue order, so at most
  // issued - PT·(t+1) may stay in flight (a smaller count only waits longer).
  auto wait_tile = [&](int t) ATTN_INLINE {
    const int pending = issued - PT * (t + 1);
    if (pending <= 0) wait_vm<0>();
    else if (pending == 1) wait_vm<1>();
    else if (pending == 2) wait_vm<2>();
    else if (pending == 3) wait_vm<3>();
    else if (pending == 4) wait_vm<4>();
    else if (pending == 5) wait_vm<5>();
    else if (pending == 6) wait_vm<6>();
    else if (pending == 7) wait_vm<7>();
    else wait_vm<8>();
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
        v_rd[dt][p] = Cfg::VREG + r * ROWB + ((lc ^ swz_v<D>(r)) * 16) + 8 * (j & 1);
      }
    }
  }

  f32x16 oacc[NB][DT];
  // Row sums l.  At d=64, where the vector unit sets the pace, on the matrix
  // cores: one 16x16x32 MFMA per 16-key k-step with the probabilities as its B
  // operand.  Read that way, lane i's 8 values sit in column i % 16 at
  // k = 8·(i / 16) .. +7, so column c mixes query c (lane groups 0 and 2, the
  // two key halves) and query c + 16 (groups 1 and 3).  The A operand `ones`
  // sums groups {0, 2} into output rows 0 and 8 and groups {1, 3} into rows 4
  // and 12; output row 4·(i / 16) lands in lane i, so element 0 of every
  // lane's accumulator is its own query's row sum (lanes q and q + 32 alike).
  // The other elements stay 0.  At d=128 the extra MFMAs and registers cost
  // more than the vector work they save (measured), and l is summed from the
  // packed probabilities by v_dot2 in the vector step instead.
  constexpr bool kMatSum = D == 64;
  float l_run[NB];  // d=128: this lane's half of the row sum (16 of every 32 keys)
  u32x4 ones;
  {
    const int m = lane & 15, g = lane >> 4;
    const bool on = (g & 1) ? (m == 4 || m == 12) : (m == 0 || m == 8);
    const uint32_t w = on ? T::kOnePair : 0u;
    ones = u32x4{w, w, w, w};
  }
  f32x4 lsum[NB];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    lsum[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run[blk] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[blk][dt][e] = 0.f;
  }

  // Operands read during the matrix step before the one that uses them.
  u32x4 kf[KK];      // K of the next score subtile
  u32x4 vf[DT][2];   // V of the next P·V subtile, per output tile and 16-key k-step
  f32x16 s[NB];      // scores of one subtile: s[blk][e] is key 16·(e>>3) + 8·half + (e&7)
                     // of the subtile against query qw + 32·blk + l32
  u32x4 pf[NB][2];   // probabilities of one subtile, B operands of P·V

  // LDS buffer ("stage") of a tile: an int, or a std::integral_constant where
  // the loop is unrolled so that the stage offset folds into the instructions'
  // 16-bit address offsets.  Buffer b holds its K tile at b·TILE and its V tile
  // at VREG + b·TILE, so every such offset stays below 64 KB.
  auto subtile = [&](auto stg, int sb) ATTN_INLINE { return lds + (int)stg * Cfg::TILE + sb * 32 * ROWB; };
  auto next_stage = [&](auto stg) ATTN_INLINE {
    if constexpr (std::is_same<decltype(stg), int>::value)
      return stg + 1 == S ? 0 : stg + 1;
    else
      return std::integral_constant<int, (decltype(stg)::value + 1) % S>{};
  };
  auto load_k = [&](auto stg, int sb) ATTN_INLINE {
    const char* st = subtile(stg, sb);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kf[kk] = lds_read16(st, k_rd[kk]);
  };
  auto load_v = [&](auto stg, int sb) ATTN_INLINE {
    const char* st = subtile(stg, sb);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x2 va = lds_read_tr16(st + ks * 16 * ROWB, v_rd[dt][0]);
        const u32x2 vb = lds_read_tr16(st + ks * 16 * ROWB, v_rd[dt][1]);
        vf[dt][ks] = u32x4{va[0], va[1], vb[0], vb[1]};
      }
  };

  auto qk = [&]() ATTN_INLINE {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[blk][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) s[blk] = T::mfma32(kf[kk], qf[blk][kk], s[blk]);
  };

  // scores of the staged K operand while the K operand of subtile sb of the
  // tile in buffer stg is read into the same registers, each after its last use
  auto qk_load_k = [&](auto stg, int sb) ATTN_INLINE {
    const char* st = subtile(stg, sb);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[blk][e] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) s[blk] = T::mfma32(kf[kk], qf[blk][kk], s[blk]);
      kf[kk] = lds_read16(st, k_rd[kk]);
      __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  auto rowsum = [&]() ATTN_INLINE {
    if constexpr (!kMatSum) return;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) lsum[blk] = T::mfma16(ones, pf[blk][ks], lsum[blk]);
  };
  auto pv = [&]() ATTN_INLINE {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) oacc[blk][dt] = T::mfma32(vf[dt][ks], pf[blk][ks], oacc[blk][dt]);
    rowsum();
  };
  // P·V of the staged V operand while the V operand of subtile sb of tile t is
  // read into the same registers, each fragment right after its last use
  auto pv_load_v = [&](auto stg, int sb) ATTN_INLINE {
    const char* st = subtile(stg, sb);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) oacc[blk][dt] = T::mfma32(vf[dt][ks], pf[blk][ks], oacc[blk][dt]);
        const u32x2 va = lds_read_tr16(st + ks * 16 * ROWB, v_rd[dt][0]);
        const u32x2 vb = lds_read_tr16(st + ks * 16 * ROWB, v_rd[dt][1]);
        vf[dt][ks] = u32x4{va[0], va[1], vb[0], vb[1]};
        __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);  // the MFMA(s) ...
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // ... then the two reads
      }
    rowsum();
  };  // The next V operand is read between the P·V MFMAs at d=128; at d=64, whose
  // vector steps are the longer ones, after all of the step's MFMAs (measured).
  auto pv_then_load_v = [&](auto stg, int sb) ATTN_INLINE {
    if (D == 64) {
      pv();
      __builtin_amdgcn_sched_barrier(0);
      load_v(stg, sb);
    } else {
      pv_load_v(stg, sb);
    }
  };

  // probabilities of the subtile starting at key s0, rounded to the storage
  // type as the B operands of P·V (and, at d=64, of the row-sum MFMAs).  The
  // exponentials use the row's current reference m (the largest row maximum
  // seen when it was last raised), kept as neg_ref = -m.  The reference is
  // raised -- to the row maximum so far, with o and l rescaled by
  // exp2(m - m_new) -- and the subtile recomputed only when some probability
  // of the wave grows too large, or on a row's first subtile with a visible
  // key (no reference yet).  Every probability used is therefore bounded and
  // the row maximum at most 8 above the reference, so nothing overflows or
  // loses precision; o and l share the reference, so o/l is the same either
  // way.  The raise test:
  //   d=64  -- some probability above 2^8.  The lane's largest rounded
  //            probability comes from a packed-max tree over the pairs (their
  //            bit patterns order like their values), lands in the high half
  //            of a 32-bit word and is compared with 256 there, as unsigned
  //            words.  A row without a reference holds neg_ref = +inf: its
  //            exponentials are +inf (visible keys) or NaN (masked ones), whose
  //            patterns -- NaN of either sign included -- pass the threshold.
  //   d=128 -- the lane's 16 probabilities summing past 2^8, the sum taken
  //            with the row sum itself (two v_dot2 chains, one of them starting
  //            from l); `lim` = -1 forces the raise while the row has no
  //            reference (neg_ref = 0 then).
  // The raise runs after the barrier that ends the vector step, at the start
  // of the wave's next matrix step and before its first MFMA, so the wave
  // reaches the barrier without waiting for the test (which hangs on the
  // whole exponential chain).  It touches no LDS and no other wave's data,
  // and the scores it needs are still in registers.
  constexpr uint32_t kRaiseLimit = (T::kBits256 << 16) | 0xFFFFu;
  constexpr float kRescaleSum = 256.f;
  float neg_ref[NB], lim[NB];
  float lnew[NB];  // d=128: the row sums with the latest subtile; d=64: its largest probability
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    neg_ref[blk] = kMatSum ? __builtin_huge_valf() : 0.f;
    lim[blk] = -1.f;
  }
  // the lane's 16 rounded probabilities into pf[blk]; returns, at d=64, their
  // largest (high half of the word), at d=128 acc plus their sum
  auto probs = [&](int blk, float nref, float acc) ATTN_INLINE {
    float ps[2] = {acc, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = fast_exp2(fmaf(s[blk][8 * ks + 2 * i], c, nref));
        const float a1 = fast_exp2(fmaf(s[blk][8 * ks + 2 * i + 1], c, nref));
        pf[blk][ks][i] = T::pack2(a0, a1);
        if constexpr (!kMatSum) ps[i & 1] = T::add_pair(ps[i & 1], pf[blk][ks][i]);
      }
    if constexpr (kMatSum) {
      uint32_t t = pk_max3_16(pf[blk][0][0], pf[blk][0][1], pf[blk][0][2]);
      t = pk_max3_16(t, pf[blk][0][3], pf[blk][1][0]);
      t = pk_max3_16(t, pf[blk][1][1], pf[blk][1][2]);
      t = pk_max3_16(t, pf[blk][1][3], t);
      return __uint_as_float(pk_max3_16<true>(t, t, t));
    } else {
      return ps[0] + ps[1];
    }
  };
  auto raise_ref = [&]() ATTN_INLINE {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      float m3[6];
#pragma unroll
      for (int i = 0; i < 5; ++i) m3[i] = fmaxf(fmaxf(s[blk][3 * i], s[blk][3 * i + 1]), s[blk][3 * i + 2]);
      m3[5] = s[blk][15];
      const float mx = fmaxf(fmaxf(fmaxf(m3[0], m3[1]), m3[2]), fmaxf(fmaxf(m3[3], m3[4]), m3[5]));
      // the current reference (-inf while the row has none)
      const float m_old = kMatSum ? (neg_ref[blk] == __builtin_huge_valf() ? kNegInf : -neg_ref[blk])
                                  : (lim[blk] < 0.f ? kNegInf : -neg_ref[blk]);
      const float m_new = fmaxf(m_old, max_xor32(mx) * c);
      const float ref = m_new == kNegInf ? 0.f : m_new;  // a row with no live key stays empty
      const float alpha = fast_exp2(m_old - ref);
      if constexpr (kMatSum) lsum[blk][0] *= alpha;
      else l_run[blk] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[blk][dt] *= alpha;
      if constexpr (kMatSum) {
        neg_ref[blk] = m_new == kNegInf ? __builtin_huge_valf() : -ref;
      } else {
        neg_ref[blk] = -ref;
        lim[blk] = m_new == kNegInf ? -1.f : kRescaleSum;
      }
      lnew[blk] = probs(blk, -ref, l_run[blk]);
    }
  };
  auto softmax = [&](int s0) ATTN_INLINE -> bool {
    if (s0 + 32 > nk || (CAUSAL && s0 + 31 > qw + off) ||
        (window > 0 && s0 <= qw + 32 * NB - 1 + off - window)) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int qlim = qw + 32 * blk + l32 + off;  // this row's position: the last key it sees if causal
        if constexpr (VARLEN) {
          // visible keys of this row: [lo, hi]; one unsigned range test per score
          // (key - lo wraps past span for keys below lo; an empty range masks all)
          const int hi = CAUSAL ? min(qlim, nk - 1) : nk - 1;
          const int lo = window > 0 ? max(qlim - window + 1, 0) : 0;
          const uint32_t lo_u = hi >= lo ? (uint32_t)lo : 0x80000000u;
          const uint32_t span = hi >= lo ? (uint32_t)(hi - lo) : 0u;
          const uint32_t base = (uint32_t)(s0 + 8 * half) - lo_u;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (base + (uint32_t)(16 * (e >> 3) + (e & 7)) > span) s[blk][e] = kNegInf;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = s0 + 16 * (e >> 3) + 8 * half + (e & 7);
            if (key >= nk || (CAUSAL && key > qlim)) s[blk][e] = kNegInf;
          }
        }
      }
    }
    if (alibi) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const float base = alibi_raw * (float)(s0 + 8 * half - (qw + 32 * blk + l32 + off));
#pragma unroll
        for (int e = 0; e < 16; ++e) s[blk][e] += fmaf(alibi_raw, (float)(16 * (e >> 3) + (e & 7)), base);
      }
    }
    bool grow = false;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      lnew[blk] = probs(blk, neg_ref[blk], l_run[blk]);
      if constexpr (kMatSum)
        grow |= __float_as_uint(lnew[blk]) > kRaiseLimit;  // also for inf or NaN
      else
        grow |= !(lnew[blk] - l_run[blk] <= lim[blk]);  // the subtile's sum
    }
    return __builtin_amdgcn_ballot_w64(grow) != 0;
  };
  // The end of a vector step: its barrier, then the raise if the test asked
  // for one, then (d=128) the new row sums take effect.
  auto vector_step_end = [&](bool raise, auto wait_lds) ATTN_INLINE {
    step_end<decltype(wait_lds)::value>();
    if (__builtin_expect(raise, 0)) {
      raise_ref();
      // the raised state in place of the old (without these pins the register
      // allocator copies every output accumulator on the common path)
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) pin(oacc[blk][dt]);
        if constexpr (kMatSum) pin(lsum[blk]);
        pin(pf[blk][0]);
        pin(pf[blk][1]);
      }
    }
    if constexpr (!kMatSum) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) l_run[blk] = lnew[blk];
    }
  };

  // results of a vector step (probabilities and running statistics) and of a
  // matrix step (scores and output accumulators)
  auto pin_vector_step = [&]() ATTN_INLINE {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      pin(pf[blk][0]);
      pin(pf[blk][1]);
      pin(neg_ref[blk]);
      if constexpr (!kMatSum) {
        pin(l_run[blk]);
        pin(lnew[blk]);
        pin(lim[blk]);
      }
    }
  };
  auto pin_matrix_step = [&]() ATTN_INLINE {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      pin(s[blk]);
      if constexpr (kMatSum) pin(lsum[blk]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) pin(oacc[blk][dt]);
    }
  };

  // ---- the steps of one wave, for subtiles u = 2t (sb 0) and 2t+1 (sb 1) of tile t:
  //   step 0      matrix  scores of subtile 0 (K of 0 read first); read K of 1, V of 0
  //   step 4t+1   vector  softmax of 2t
  //   step 4t+2   matrix  scores of 2t+1, P·V of 2t;   read K of 2t+2, V of 2t+1
  //   step 4t+3   vector  softmax of 2t+1
  //   step 4t+4   matrix  scores of 2t+2, P·V of 2t+1; read K of 2t+3, V of 2t+2
  // Each operand is read into its registers right after the MFMA that last
  // used them, so the reads overlap the MFMAs; tile t is read by steps
  // 4t-2 .. 4t+2 (0 .. 2 for tile 0).  Every step ends at a workgroup barrier.
  // Group 1 passes one extra barrier first, so it runs each step one phase
  // after group 0: on every SIMD one wave is in a matrix step while the other
  // is in a vector step.
  //
  // Tiles 0 .. S-1 are fetched up front.  Tile t+S-1 (t >= 1) is fetched at the
  // start of vector steps 4t+1 and 4t+3, half of its transfers each; its buffer
  // last held tile t-1, whose final read (group 1, step 4t-2) has returned by
  // the end of group 1's vector step 4t-1, i.e. before the barrier that opens
  // group 0's step 4t+1.  Each wave waits for its transfers of tile t+1 at the
  // end of step 4t, before the barriers that precede group 0's first read of
  // it (step 4t+2).
  static_assert(S >= 3, "the fetch schedule needs three tile buffers");
  static_assert(PT % 2 == 0 && PT <= 4, "transfers split evenly over the two vector steps of a tile");
  fetch_tile();
  wait_vm<0>();  // Q operands and tile 0
  step_end<true>();
#pragma unroll
  for (int t = 1; t < S; ++t)  // in flight during the first steps
    if (t < nkt) fetch_tile();
  if (grp == 1) step_end<true>();

  load_k(std::integral_constant<int, 0>{}, 0);
  qk_load_k(std::integral_constant<int, 0>{}, 1);
  load_v(std::integral_constant<int, 0>{}, 0);
  if (nkt > 1) wait_tile(1);
  pin_matrix_step();
  step_end<false>();
  // Transfers of the tile being fetched, issued at the start of a vector step
  // (measured: issued inside a matrix step they can hold up its MFMAs).  The
  // cursor then advances in the matrix step after the second half, whose
  // wave has time to spare at its barrier.
  auto fetch_half = [&](bool fetch, auto h) ATTN_INLINE {
    __builtin_amdgcn_sched_barrier(0);
    if (fetch) static_for<decltype(h)::value * PT / 2, (decltype(h)::value + 1) * PT / 2>(fetch_part);
    __builtin_amdgcn_sched_barrier(0);
  };
  // one tile; the last one has no successor to read or score
  auto tile_steps = [&](int t, auto stg, auto last_tag) ATTN_INLINE {
    constexpr bool LAST = decltype(last_tag)::value;
    const bool fetch = t >= 1 && t + S - 1 < nkt;
    // step 4t+1: softmax of subtile 2t
    fetch_half(fetch, std::integral_constant<int, 0>{});
    const bool raise0 = softmax(key0 + 64 * t);
    pin_vector_step();
    vector_step_end(raise0, std::integral_constant<bool, D == 128>{});  // (measured: d=64 -0.7 %, d=128 +0.2 %)
    // step 4t+2: scores of 2t+1, P·V of 2t; K of 2t+2, V of 2t+1
    if (LAST) qk(); else qk_load_k(next_stage(stg), 0);
    pv_then_load_v(stg, 1);
    pin_matrix_step();
    step_end<false>();
    // step 4t+3: softmax of 2t+1 (the last tile: the next item's Q is read first)
    if constexpr (LAST && !CAUSAL && !VARLEN) {
      if (next_bid >= 0) prefetch_q();
    }
    fetch_half(fetch, std::integral_constant<int, 1>{});
    const bool raise1 = softmax(key0 + 64 * t + 32);
    pin_vector_step();
    vector_step_end(raise1, std::true_type{});
    // step 4t+4: scores of 2t+2, P·V of 2t+1; K of 2t+3, V of 2t+2; tile t+2 landed
    if (LAST) {
      pv();
    } else {
      qk_load_k(next_stage(stg), 1);
      pv_then_load_v(next_stage(stg), 0);
      // tiles 0 .. min(t+3, nkt-1) are issued by now (tile t+3 during this tile's vector
      // steps), so tile t+2 has landed once at most the PT·(S-3) transfers after it are in flight
      if (t + 2 < nkt) {
        if (t + S <= nkt) wait_vm<PT * (S - 3)>();
        else wait_vm<0>();
      }
      if (fetch) fetch_advance();
    }
    pin_matrix_step();
    step_end<false>();
  };
  // groups of S tiles (none of them the last) with compile-time stages, then
  // the remaining tiles with run-time stages
  auto group = [&](auto self, int t0, auto j) ATTN_INLINE {
    tile_steps(t0 + decltype(j)::value, j, std::false_type{});
    if constexpr (decltype(j)::value + 1 < S) self(self, t0, std::integral_constant<int, decltype(j)::value + 1>{});
  };
  int t = 0;
  for (; t + S < nkt; t += S) group(group, t, std::integral_constant<int, 0>{});
  for (; t + 1 < nkt; ++t) tile_steps(t, t % S, std::false_type{});
  tile_steps(nkt - 1, (nkt - 1) % S, std::true_type{});
  if (grp == 0) step_end<true>();

  // ---- epilogue: O = o / l, rounded to the storage type, written once.
  // Every LDS read and tile transfer has completed before the barrier just
  // passed, so the tile buffers are free: each wave stages its rows (32·NB of
  // them, contiguous in O) in its own 8 KB of LDS and writes them back as
  // whole 1 KB runs instead of 16-byte pieces of 32 rows per instruction.
  float inv[NB];
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    // d=64: both key halves (lanes q and q + 32 hold the same sum); d=128: add the other half
    const float l_tot = kMatSum ? lsum[blk][0] : sum_xor32(l_run[blk]);
    inv[blk] = l_tot > 0.f ? 1.f / l_tot : 0.f;
  }
  constexpr uint32_t WAVE_OUT = 32 * NB * ROWB;  // bytes of this wave's output rows
  static_assert(WAVE_OUT == 8192 && Cfg::WAVES * WAVE_OUT <= Cfg::LDS, "output staging fits the tile buffers");
  char* ostage = lds + wave * WAVE_OUT;
  // 16-byte chunk c of staged row r sits at chunk c ^ oswz(r): the 32 lanes of
  // a half-wave write 8-byte halves of one chunk column across 16 rows, and
  // read 16-byte chunks of whole rows, both without bank conflicts
  auto oswz = [](int r) ATTN_INLINE { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int r = 32 * blk + l32;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int eh = 0; eh < 4; ++eh) {  // columns 32·dt + 8·eh + 4·half .. +3 = half of chunk 4·dt + eh
        const u32x2 w = {T::pack2(oacc[blk][dt][4 * eh + 0] * inv[blk], oacc[blk][dt][4 * eh + 1] * inv[blk]),
                         T::pack2(oacc[blk][dt][4 * eh + 2] * inv[blk], oacc[blk][dt][4 * eh + 3] * inv[blk])};
        *reinterpret_cast<u32x2*>(ostage + r * ROWB + (((4 * dt + eh) ^ oswz(r)) * 16) + 8 * half) = w;
      }
  }
#pragma unroll
  for (int i = 0; i < (int)(WAVE_OUT / 1024); ++i) {
    const int byte = i * 1024 + lane * 16;
    const int r = byte / ROWB, ch = (byte % ROWB) / 16;
    const u32x4 x = lds_read16(ostage, r * ROWB + ((ch ^ oswz(r)) * 16));
    const int qrow = qw + r;
    if (qrow < nq) gstore16(o + qo_base + (size_t)qrow * q_stride + ch * 16, x);
  }
}

// The square non-causal kernels run persistently: workgroup j takes items j,
// j + G, j + 2G, ... (G = gridDim.x, a multiple of 8, so every item stays on
// the XCD the mapping above gives it), reading each next item's Q during the
// current one.  The other kernels take one item per workgroup.
template <class T, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_fwd_kernel(
    const char* __restrict__ q, const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ o,
    int batch, int hq, int hkv, int n, float c, int num_q_tiles, VarlenArgs vl, MaskArgs mk, int items) {
  u32x4 qf[PrefillCfg<D>::NB][D / 16];
  if constexpr (!CAUSAL && !VARLEN) {
    bool have_q = false;
    for (int bid = blockIdx.x; bid < items; bid += (int)gridDim.x) {
      const int next = bid + (int)gridDim.x < items ? bid + (int)gridDim.x : -1;
      prefill_item<T, D, CAUSAL, VARLEN>(bid, next, qf, have_q, q, k, v, o, batch, hq, hkv, n, c, num_q_tiles, vl,
                                         mk);
      have_q = next >= 0;
      __syncthreads();  // the output staging in LDS is read before the next item's tiles land there
    }
  } else {
    prefill_item<T, D, CAUSAL, VARLEN>(blockIdx.x, -1, qf, false, q, k, v, o, batch, hq, hkv, n, c, num_q_tiles, vl,
                                       mk);
  }
}

// Compute units of the device `stream` runs on (cached per device; 0 if unknown).
static int compute_units(hipStream_t stream) {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) return 0;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0 && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    cached[dev].store(cus, std::memory_order_relaxed);
  return cus > 0 ? cus : 0;
}

template <class T, int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_prefill_t(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                                   int n, float scale, VarlenArgs vl, MaskArgs mk, hipStream_t stream) {
  using Cfg = PrefillCfg<D>;
  const int tiles = (n + Cfg::BR - 1) / Cfg::BR;
  // varlen: 8 XCDs x (units of the fullest XCD) x query heads per unit x tiles
  const long long blocks = VARLEN ? 8LL * ((batch * hkv + 7) / 8) * (hq / hkv) * tiles : (long long)tiles * hq * batch;
  // square non-causal kernels with heads grouped per XCD: one persistent
  // workgroup per compute unit (a workgroup fills a compute unit's LDS and registers)
  long long grid = blocks;
  if (!CAUSAL && !VARLEN && (batch * hq) % 8 == 0) {
    const long long cus = compute_units(stream) / 8 * 8;
    if (cus > 0 && blocks > cus) grid = cus;
  }
  prefill_fwd_kernel<T, D, CAUSAL, VARLEN><<<dim3((unsigned)grid), dim3(64 * Cfg::WAVES), 0, stream>>>(
      static_cast<const char*>(q), static_cast<const char*>(k), static_cast<const char*>(v), static_cast<char*>(o),
      batch, hq, hkv, n, scale * kLog2e, tiles, vl, mk, (int)blocks);
  return hipGetLastError();
}

template <class T, int D, bool VARLEN>
static hipError_t launch_prefill_d(const void* q, const void* k, const void* v, void* o, int batch, int hq, int hkv,
                                   int n, float scale, bool causal, VarlenArgs vl, MaskArgs mk, hipStream_t stream) {
  return causal ? launch_prefill_t<T, D, true, VARLEN>(q, k, v, o, batch, hq, hkv, n, scale, vl, mk, stream)
                : launch_prefill_t<T, D, false, VARLEN>(q, k, v, o, batch, hq, hkv, n, scale, vl, mk, stream);
}

template <bool VARLEN>
static hipError_t launch_prefill_any(const void* q, const void* k, const void* v, void* o, bool bf16, int batch,
                                     int hq, int hkv, int n, int d, float scale, bool causal, VarlenArgs vl,
                                     MaskArgs mk, hipStream_t stream) {
  if (bf16)
    return d == 64
               ? launch_prefill_d<Bf16, 64, VARLEN>(q, k, v, o, batch, hq, hkv, n, scale, causal, vl, mk, stream)
               : launch_prefill_d<Bf16, 128, VARLEN>(q, k, v, o, batch, hq, hkv, n, scale, causal, vl, mk, stream);
  return d == 64 ? launch_prefill_d<F16, 64, VARLEN>(q, k, v, o, batch, hq, hkv, n, scale, causal, vl, mk, stream)
                 : launch_prefill_d<F16, 128, VARLEN>(q, k, v, o, batch, hq, hkv, n, scale, causal, vl, mk, stream);
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, void* o, bool bf16, int batch, int hq,
                          int hkv, int n, int d, float scale, bool causal, hipStream_t stream) {
  return launch_prefill_any<false>(q, k, v, o, bf16, batch, hq, hkv, n, d, scale, causal,
                                   VarlenArgs{nullptr, nullptr, 0, 0, 0}, MaskArgs{0, nullptr}, stream);
}

hipError_t launch_prefill_varlen(const void* q, const void* k, const void* v, void* o, const int* cu_q,
                                 const int* cu_k, int total_q, int total_k, int max_q, int max_k, bool bf16, int batch,
                                 int hq, int hkv, int d, float scale, bool causal, int window, const float* alibi,
                                 hipStream_t stream) {
  return launch_prefill_any<true>(q, k, v, o, bf16, batch, hq, hkv, max_q, d, scale, causal,
                                  VarlenArgs{cu_q, cu_k, total_q, total_k, max_k}, MaskArgs{window, alibi}, stream);
}

}  // namespace attn
