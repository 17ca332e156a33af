// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Vector types, 128-bit memory access, the bf16/fp16 matrix-core (MFMA)
// instructions used for the two contractions Q·Kᵀ and P·V, the LDS transpose
// read used to feed V to the matrix cores, and fp32 -> bf16/fp16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Storage element tags.  Both are 16-bit; they differ in the MFMA opcode and
// in how fp32 is rounded back to storage.
struct Bf16 {
  static constexpr uint32_t kOnePair = 0x3F803F80u;  // (1.0, 1.0)
  static constexpr uint32_t kBits256 = 0x4380u;      // 256.0
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint32_t, v);
  }
  // acc + lo + hi of a packed pair (v_dot2_f32_bf16 against (1, 1))
  static __device__ __forceinline__ float add_pair(float acc, uint32_t pair) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
  }
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  }
};

struct F16 {
  static constexpr uint32_t kOnePair = 0x3C003C00u;  // (1.0, 1.0)
  static constexpr uint32_t kBits256 = 0x5C00u;      // 256.0
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    f16x2 v = {(_Float16)a, (_Float16)b};  // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float add_pair(float acc, uint32_t pair) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
  }
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  }
};

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// 16-byte global load / store (global_load_dwordx4 / global_store_dwordx4).
__device__ __forceinline__ u32x4 gload16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void gstore16(void* p, u32x4 x) { *reinterpret_cast<u32x4*>(p) = x; }
__device__ __forceinline__ void gstore8(void* p, u32x2 x) { *reinterpret_cast<u32x2*>(p) = x; }

// Buffer resource over [base, base + bytes): raw buffer loads through it read
// 0 for any offset at or past `bytes`, so tails need no branches and nothing
// past the range is ever touched.  The resource lives in scalar registers and
// must be wave-uniform.
typedef __amdgpu_buffer_rsrc_t bufres;
constexpr int kBufferFlags = 0x00020000;  // gfx9 buffer descriptor word 3: 32-bit data format
__device__ __forceinline__ bufres make_bufres(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}
__device__ __forceinline__ u32x4 bload16(bufres r, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0));
}

// Buffer-load-to-LDS of 16 bytes per lane: lane i's bytes (from voffset in the
// buffer described by `rsrc`, 0 past its end) land at LDS byte address
// `lds_base + OFF + 16·i`.  `lds_base` must be wave-uniform.
//
// Issued as inline assembly on purpose.  The compiler cannot tell which LDS
// bytes a DMA writes, so after one it makes the next LDS read of ANY address
// wait for the DMA to finish -- which serialises a prefetch of a later tile
// with the reads of the current one.  Callers instead wait explicitly
// (vmcnt(0) and a barrier) before reading the destination; the compiler sees
// only a memory-clobbering statement and keeps other memory operations in
// order around it.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 bufres_words(const void* base, uint32_t bytes) {
  // the words must sit in scalar registers even when the compiler computed a
  // (wave-uniform) input with vector instructions
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane((int)bytes), kBufferFlags};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const ATTN_LDS char*)p;
}
// The destination is `lds_base + OFF`, added straight into M0.
template <uint32_t OFF>
__device__ __forceinline__ void dma16_to_lds(i32x4 rsrc, uint32_t voffset, uint32_t lds_base) {
  // Wait states before the load: a buffer load must not read an SGPR that a
  // vector instruction wrote fewer than 5 wait states earlier (the resource
  // words come from v_readfirstlane, and the compiler may reload spilled
  // scalars with v_readlane right before this statement), and the compiler
  // does not check that hazard for inline assembly -- so the M0 write and
  // s_nop 3 give 5 here, whatever precedes (with fewer, a v_readlane two wait
  // states before a load has been seen to give wrong results).  The M0 write
  // needs one of them too.  M0 is not listed as clobbered (the compiler
  // rejects that for a reserved register); the compiler itself writes M0
  // right before any instruction of its own that reads it, so nothing it
  // holds there lives across this one.  The scalar add also writes the
  // condition code SCC, which must be listed: otherwise the compiler may
  // keep a carry or a comparison in SCC across the statement (a 64-bit
  // pointer increment split around it lost its carry that way).
  asm volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 3\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset),
      "s"(rsrc), "s"(lds_base), "n"(OFF)
      : "memory", "scc");
}
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// LDS access at a byte offset from an LDS base pointer.
__device__ __forceinline__ u32x4 lds_read16(const char* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(char* base, uint32_t off, u32x4 x) {
  *reinterpret_cast<u32x4*>(base + off) = x;
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j names 8 bytes: columns 4·(j%4) .. 4·(j%4)+3 of row j/4 of a 4 x 16
// block of 16-bit elements.  Lane i of the group receives column i of that
// block: its 4 rows, in row order.  Reading V (rows = keys, columns = head
// dimension) this way hands each lane 4 consecutive keys of one column, which
// is the k-major operand layout of the matrix instructions.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* base, uint32_t off) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(base + off));
  return __builtin_bit_cast(u32x2, r);
}

// Element-wise maximum of three packed pairs of 16-bit floats (v_pk_maximum3_f16).
// Used on non-negative bf16 or fp16 bit patterns below 0x7C00, whose order as
// fp16 values is the order of their bits, so it serves both types.  HI_FROM_LO
// makes the high result take max(a.hi, b.lo, c.hi): the high half then holds
// the largest of all four.
template <bool HI_FROM_LO = false>
__device__ __forceinline__ uint32_t pk_max3_16(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  if (HI_FROM_LO)
    asm("v_pk_maximum3_f16 %0, %1, %2, %3 op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  else
    asm("v_pk_maximum3_f16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// exp2 on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane reductions without LDS.  v_permlane32_swap exchanges rows 2-3
// (lanes 32..63) of its first operand with rows 0-1 (lanes 0..31) of its
// second; given the same value twice it returns (lower half, lower half) and
// (upper half, upper half), so combining the pair reduces lane l with lane
// l^32 and leaves the same bits in both.  v_permlane16_swap does the same for
// rows 1/3 against rows 0/2, pairing lane l with lane l^16.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace attn
