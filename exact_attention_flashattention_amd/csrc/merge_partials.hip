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
// One workgroup of 256 threads per (sequence, head).  Each thread owns 4
// consecutive output columns; the D/4 threads of a column group form one "row
// group", and the 256/(D/4) row groups take the splits round-robin, so every
// split's o row is read with contiguous 16-byte loads.  Row-group results are
// combined through LDS.  Memory-bound: it reads S·(D+2) floats per row once.
#include "device_common.hpp"
#include "launchers.hpp"

namespace attn {

template <class T, int D>
__global__ __launch_bounds__(256) void merge_partials_kernel(const float* __restrict__ part_m,
                                                             const float* __restrict__ part_l,
                                                             const float* __restrict__ part_o, int num_splits,
                                                             void* __restrict__ out) {
  constexpr int COLS = D / 4;          // threads per row group
  constexpr int GROUPS = 256 / COLS;   // row groups
  __shared__ float red[256];
  __shared__ f32x4 acc_s[GROUPS][COLS];
  __shared__ float l_s[GROUPS];

  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;  // b * hq + h
  const float* m_ = part_m + row * num_splits;
  const float* l_ = part_l + row * num_splits;
  const float* o_ = part_o + row * (size_t)num_splits * D;

  // 1. the largest partial maximum
  float mx = kNegInf;
  for (int s = tid; s < num_splits; s += 256) mx = fmaxf(mx, m_[s]);
  red[tid] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];

  // 2. weighted sums of o and l over this row group's splits
  const int c = tid % COLS, g = tid / COLS;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  if (M != kNegInf) {
    for (int s = g; s < num_splits; s += GROUPS) {
      const float ms = m_[s];
      const float w = (ms == kNegInf) ? 0.f : fast_exp2((ms - M) * kLog2e);
      const f32x4 os = *reinterpret_cast<const f32x4*>(o_ + (size_t)s * D + 4 * c);
      acc += w * os;
      lsum += w * l_[s];
    }
  }
  acc_s[g][c] = acc;
  if (c == 0) l_s[g] = lsum;
  __syncthreads();

  // 3. combine row groups and normalise
  if (tid < COLS) {
    f32x4 tot = acc_s[0][tid];
    float l = l_s[0];
    for (int r = 1; r < GROUPS; ++r) {
      tot += acc_s[r][tid];
      l += l_s[r];
    }
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    tot *= inv;
    u32x2 packed = {T::pack2(tot[0], tot[1]), T::pack2(tot[2], tot[3])};
    gstore8(reinterpret_cast<char*>(out) + (row * D + 4 * tid) * 2, packed);
  }
}

template <class T, int D>
static hipError_t launch_merge_t(const float* pm, const float* pl, const float* po, int rows, int num_splits,
                                 void* out, hipStream_t stream) {
  merge_partials_kernel<T, D><<<dim3(rows), dim3(256), 0, stream>>>(pm, pl, po, num_splits, out);
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
