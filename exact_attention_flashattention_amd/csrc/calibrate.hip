// On-device ceilings that a kernel's roofline fraction can also be quoted
// against, beside the published peaks: a back-to-back bf16 MFMA loop (the
// matrix-core rate this chip sustains under full load, clock throttling
// included) and a streaming read of a large buffer (the HBM read rate a plain
// kernel reaches).  Neither is part of the attention path.
#include "device_common.hpp"
#include "launchers.hpp"

namespace attn {

// Each wave runs `iters` rounds of four independent 32x32x16 bf16 MFMA chains
// on register operands (4 · 32768 FLOP per round).  The operands come from the
// thread index so nothing folds; the sums are stored so nothing is dropped.
__global__ __launch_bounds__(256) void calib_mfma_kernel(float* __restrict__ out, int iters) {
  u32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = Bf16::pack2((float)(threadIdx.x + i) * 1e-3f, 0.5f);
    b[i] = Bf16::pack2(0.25f, (float)i * 1e-2f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = Bf16::mfma32(a, b, c0);
    c1 = Bf16::mfma32(a, b, c1);
    c2 = Bf16::mfma32(a, b, c2);
    c3 = Bf16::mfma32(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Grid-stride read of n16 16-byte chunks, each once; the XOR of what a thread
// read is stored only if it equals a value it practically never does, so the
// kernel writes (almost) nothing.  (Measured on a 1 GiB buffer: unrolling to
// four or eight independent loads per thread, or non-temporal loads, does not
// raise the rate.)
__global__ __launch_bounds__(256) void calib_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                         u32x4* __restrict__ out) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) acc ^= p[i];
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) out[threadIdx.x] = acc;
}

hipError_t launch_calib_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  calib_mfma_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(out, iters);
  return hipGetLastError();
}

hipError_t launch_calib_read(const void* buf, size_t bytes, void* scratch, int blocks, hipStream_t stream) {
  calib_read_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(static_cast<const u32x4*>(buf), bytes / 16,
                                                                       static_cast<u32x4*>(scratch));
  return hipGetLastError();
}

}  // namespace attn
