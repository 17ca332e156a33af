// Merge of split-K partial states (m, l, o) into the normalised output.
//
// For one (sequence, query head) the partials of all splits combine by
// m = max_s m_s, l = sum_s l_s·e^(m_s − m), o = sum_s o_s·e^(m_s − m), O = o/l:
// the two-state merge rule of "Maths" on "Attention kernels" applied across
// all splits at once (it is associative and commutative, "correct for any
// block order" in "02 · The insight" of "Quantized kernels").  A partial with
// m_s = −inf saw no keys and gets weight 0 -- the guard of that page's "Code"
// section -- and a row with no keys at all is written as 0.
//
// Launch shape: 256 threads per workgroup; each thread owns 4 consecutive
// output columns of one split group, and the split groups take the splits
// round-robin, so every split's o row is read with contiguous 16-byte loads,
// several in flight per thread.  Each split group folds its splits against
// its own maximum in registers, then the groups are merged in LDS by the
// same rule (in a fixed pairwise tree when there are many groups) -- one
// round trip to memory.  A workgroup covers COLS output columns: all D when there are
// many rows, 32 or 16 when few rows would leave most of the GPU idle (16 for
// many splits, so each thread reads at most a few of them).  Reads
// S·(D+2) floats per row once; with few rows it is bound by memory latency,
// so each split group folds its splits with a running maximum, which keeps
// all of a thread's loads independent.
#include "device_common.hpp"
#include "launchers.hpp"

namespace attn {

template <class T, int D, int COLS>
__global__ __launch_bounds__(256) void merge_partials_kernel(const float* __restrict__ part_m,
                                                             const float* __restrict__ part_l,
                                                             const float* __restrict__ part_o, int num_splits,
                                                             void* __restrict__ out) {
  constexpr int QUADS = COLS / 4;       // threads per split group
  constexpr int GROUPS = 256 / QUADS;   // split groups
  constexpr int CB = D / COLS;          // workgroups per row
  __shared__ f32x4 acc_s[GROUPS][QUADS];
  __shared__ float l_s[GROUPS], m_s[GROUPS];

  const int tid = threadIdx.x;
  const size_t row = blockIdx.x / CB;  // b * hq + h
  const int col0 = (blockIdx.x % CB) * COLS;
  const int c = tid % QUADS, g = tid / QUADS;
  const int col = col0 + 4 * c;
  const float* m_ = part_m + row * num_splits;
  const float* l_ = part_l + row * num_splits;
  const float* o_ = part_o + row * (size_t)num_splits * D + col;

  // 1. this group's splits, folded one by one against a running maximum mg (the
  // loads of a split do not wait for the previous split's arithmetic, so a
  // thread has several splits' loads in flight at once)
  float mg = kNegInf;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
#pragma unroll 8
  for (int s = g; s < num_splits; s += GROUPS) {
    const float ms = m_[s];
    const float ls = l_[s];
    const f32x4 os = *reinterpret_cast<const f32x4*>(o_ + (size_t)s * D);
    if (ms > mg) {  // a new maximum: rescale what is held (nothing yet while mg = -inf)
      const float a = (mg == kNegInf) ? 0.f : fast_exp2((mg - ms) * kLog2e);
      acc *= a;
      lsum *= a;
      mg = ms;
    }
    const float w = (ms == kNegInf) ? 0.f : fast_exp2((ms - mg) * kLog2e);
    acc += w * os;
    lsum += w * ls;
  }

  // 2. merge the groups.  Many groups (few rows): pairwise in a fixed tree --
  // at each level the upper half of the live groups publishes its state and
  // group g takes in group g + half (every thread of a group holds the
  // group's m and l); a level's reads and the next level's writes touch
  // disjoint slots, so one barrier per level.  Few groups: all publish, and
  // group 0 weighs them against their common maximum.  Empty states have
  // m = -inf and weight 0.
  auto take_in = [&](float mo, float lo, f32x4 ao) {
    const float M = fmaxf(mg, mo);
    const float wa = (mg == kNegInf) ? 0.f : fast_exp2((mg - M) * kLog2e);
    const float wb = (mo == kNegInf) ? 0.f : fast_exp2((mo - M) * kLog2e);
    acc = acc * wa + ao * wb;
    lsum = lsum * wa + lo * wb;
    mg = M;
  };
  if constexpr (GROUPS >= 32) {
#pragma unroll
    for (int half = GROUPS / 2; half >= 1; half /= 2) {
      if (g >= half && g < 2 * half) {
        acc_s[g][c] = acc;
        if (c == 0) {
          l_s[g] = lsum;
          m_s[g] = mg;
        }
      }
      __syncthreads();
      if (g < half) take_in(m_s[g + half], l_s[g + half], acc_s[g + half][c]);
    }
  } else {
    acc_s[g][c] = acc;
    if (c == 0) {
      l_s[g] = lsum;
      m_s[g] = mg;
    }
    __syncthreads();
    if (g == 0) {
      float M = m_s[0];
      for (int r = 1; r < GROUPS; ++r) M = fmaxf(M, m_s[r]);
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      lsum = 0.f;
      if (M != kNegInf) {
        for (int r = 0; r < GROUPS; ++r) {
          const float w = (m_s[r] == kNegInf) ? 0.f : fast_exp2((m_s[r] - M) * kLog2e);
          acc += w * acc_s[r][c];
          lsum += w * l_s[r];
        }
      }
    }
  }

  // 3. normalise (a row with no keys has l = 0 and is written as 0)
  if (g == 0) {
    const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
    acc *= inv;
    u32x2 packed = {T::pack2(acc[0], acc[1]), T::pack2(acc[2], acc[3])};
    gstore8(reinterpret_cast<char*>(out) + (row * D + col0 + 4 * c) * 2, packed);
  }
}

// Rows below this count are spread over D/32 (or, with many splits, D/16)
// workgroups each.
constexpr int kMergeFewRows = 512;

// With few rows and at least this many splits, workgroups of 16 columns.
constexpr int kMergeManySplits = 128;

template <class T, int D>
static hipError_t launch_merge_t(const float* pm, const float* pl, const float* po, int rows, int num_splits,
                                 void* out, hipStream_t stream) {
  if (rows < kMergeFewRows && num_splits >= kMergeManySplits)
    merge_partials_kernel<T, D, 16><<<dim3((unsigned)rows * (D / 16)), dim3(256), 0, stream>>>(pm, pl, po,
                                                                                          num_splits, out);
  else if (rows < kMergeFewRows)
    merge_partials_kernel<T, D, 32><<<dim3((unsigned)rows * (D / 32)), dim3(256), 0, stream>>>(pm, pl, po,
                                                                                          num_splits, out);
  else
    merge_partials_kernel<T, D, D><<<dim3((unsigned)rows), dim3(256), 0, stream>>>(pm, pl, po, num_splits, out);
  return hipGetLastError();
}

hipError_t launch_merge(const float* pm, const float* pl, const float* po, int rows, int d, int num_splits,
                        bool bf16, void* out, hipStream_t stream) {
  if (bf16) {
    return d == 64 ? launch_merge_t<Bf16, 64>(pm, pl, po, rows, num_splits, out, stream)
                   : launch_merge_t<Bf16, 128>(pm, pl, po, rows, num_splits, out, stream);
  }
  return d == 64 ? launch_merge_t<F16, 64>(pm, pl, po, rows, num_splits, out, stream)
                 : launch_merge_t<F16, 128>(pm, pl, po, rows, num_splits, out, stream);
}

}  // namespace attn
