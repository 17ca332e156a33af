// Encoder of the 4-bit KV cache read by decode_q4.hip: rows of d 16-bit
// values -> d/2 bytes of OCP MX E2M1 codes (element 2i in the low nibble of
// byte i, 2i+1 in the high nibble) and one fp32 scale per row.  This is the
// write side of "Why a quantised cache needs a fused kernel" on "Attention
// from the kernel's side": new keys and values are quantised once, as they
// enter the cache, and the attention kernel then only ever reads the codes.
//
// Per row, in fp32 and in this order (the decision of each code depends on
// the exact fp32 values, so the procedure is fixed):
//   1. if `rotated`: the Walsh-Hadamard butterflies over the element index
//      bits from bit 0 upward (lower element a, upper b -> a + b, a - b),
//      then one multiplication by `norm` = 1/sqrt(d) rounded to fp32;
//   2. scale = max|y| / 6 (1 for an all-zero row);
//   3. t = y / scale (IEEE division); the code is the nearest E2M1 magnitude
//      of |t| (0, 0.5, 1, 1.5, 2, 3, 4, 6; a tie goes to the even code) with
//      the sign bit set when t < 0.
//
// gfx950 mapping: one wavefront per row, d/64 elements per lane (lane l holds
// elements l·E .. l·E + E - 1), cross-lane butterflies and the max through
// __shfl_xor, one store of the lane's code byte (d = 128) or of a pair's byte
// (d = 64).
#include "device_common.hpp"
#include "launchers.hpp"

#include <type_traits>

namespace attn {

namespace {

// index of the nearest E2M1 magnitude to a >= 0, ties to the even index (the
// thresholds are the midpoints; '>' keeps a tie on the lower, '>=' moves it up)
__device__ __forceinline__ uint32_t e2m1_index(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

}  // namespace

template <class T, int D>
__global__ __launch_bounds__(256) void quantize_q4_kernel(const char* __restrict__ x, int rows, int rotated,
                                                          float norm, const int* __restrict__ out_rows,
                                                          int out_capacity, uint8_t* __restrict__ codes,
                                                          float* __restrict__ scales) {
  constexpr int E = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave
  const char* xr = x + (size_t)row * D * 2;
  float y[E];
  if constexpr (E == 2) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(xr + lane * 4);
    if constexpr (std::is_same<T, Bf16>::value) {
      y[0] = __uint_as_float(u << 16);
      y[1] = __uint_as_float(u & 0xffff0000u);
    } else {
      const f16x2 p = __builtin_bit_cast(f16x2, u);
      y[0] = (float)p[0];
      y[1] = (float)p[1];
    }
  } else {
    const uint16_t u = *reinterpret_cast<const uint16_t*>(xr + lane * 2);
    if constexpr (std::is_same<T, Bf16>::value) {
      y[0] = __uint_as_float((uint32_t)u << 16);
    } else {
      y[0] = (float)__builtin_bit_cast(_Float16, u);
    }
  }
  if (rotated) {
    if constexpr (E == 2) {  // element bit 0 lives inside the lane
      const float a = y[0], b = y[1];
      y[0] = a + b;
      y[1] = a - b;
    }
#pragma unroll
    for (int k = 0; k < 6; ++k) {  // element bit log2(E) + k is lane bit k
      const bool upper = (lane >> k) & 1;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float other = __shfl_xor(y[e], 1 << k);
        y[e] = upper ? other - y[e] : y[e] + other;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] *= norm;
  }
  float amax = fabsf(y[0]);
  if constexpr (E == 2) amax = fmaxf(amax, fabsf(y[1]));
#pragma unroll
  for (int k = 0; k < 6; ++k) amax = fmaxf(amax, __shfl_xor(amax, 1 << k));
  const float scale = amax > 0.f ? amax / 6.0f : 1.0f;
  uint32_t code[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float t = y[e] / scale;
    code[e] = e2m1_index(fabsf(t)) | (t < 0.f ? 8u : 0u);
  }
  const int dst = out_rows ? out_rows[row] : row;
  if (dst < 0 || dst >= out_capacity) return;  // a destination outside the cache: nothing is written
  uint8_t* cr = codes + (size_t)dst * (D / 2);
  if constexpr (E == 2) {
    cr[lane] = (uint8_t)(code[0] | (code[1] << 4));
  } else {
    const uint32_t hi = (uint32_t)__shfl_xor((int)code[0], 1);
    if ((lane & 1) == 0) cr[lane >> 1] = (uint8_t)(code[0] | (hi << 4));
  }
  if (lane == 0) scales[dst] = scale;
}

hipError_t launch_quantize_q4(const void* x, int rows, int d, bool bf16, bool rotated, float norm, const int* out_rows,
                              int out_capacity, void* codes, float* scales, hipStream_t stream) {
  const dim3 grid((rows + 3) / 4), block(256);
  const char* xs = static_cast<const char*>(x);
  uint8_t* cs = static_cast<uint8_t*>(codes);
  const int rot = rotated ? 1 : 0;
  if (bf16) {
    if (d == 64)
      quantize_q4_kernel<Bf16, 64><<<grid, block, 0, stream>>>(xs, rows, rot, norm, out_rows, out_capacity, cs, scales);
    else
      quantize_q4_kernel<Bf16, 128><<<grid, block, 0, stream>>>(xs, rows, rot, norm, out_rows, out_capacity, cs, scales);
  } else {
    if (d == 64)
      quantize_q4_kernel<F16, 64><<<grid, block, 0, stream>>>(xs, rows, rot, norm, out_rows, out_capacity, cs, scales);
    else
      quantize_q4_kernel<F16, 128><<<grid, block, 0, stream>>>(xs, rows, rot, norm, out_rows, out_capacity, cs, scales);
  }
  return hipGetLastError();
}

}  // namespace attn
