// Device-side building blocks shared by the gfx950 GEMM kernels: vector
// types, buffer resources, LDS DMA, the scaled matrix-core instruction and
// BF16 rounding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;

// Element-format codes understood by the scaled MFMA's cbsz/blgp fields.
enum : int { F_E4M3 = 0, F_E5M2 = 1, F_E2M1 = 4, F_BF16 = 32 };

// Neutral E8M0 scale (2^0) in every byte.
constexpr int E8M0_ONE_X4 = 0x7F7F7F7F;

// Buffer resource over [base, base + nbytes): loads past nbytes return 0
// (checked per dword), stores past it are dropped.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)nbytes, 0x00020000);
}

__device__ inline uint32_t clamp_records(int64_t remaining) {
  if (remaining <= 0) return 0;
  return remaining > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)remaining;
}

// The same DMA issued as inline assembly, invisible to the compiler's
// wait-count insertion: a kernel that uses it must itself wait (vmcnt) for
// the DMA before any wave reads the destination, and must not overwrite a
// destination that another wave may still read.  The resource is four SGPRs
// (base, stride 0, num_records, dword 3 as in make_rsrc).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline u32x4 rsrc4(const void *base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)base;
  return (u32x4){(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, nbytes, 0x00020000u};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// LDS byte address of a __shared__ object (32-bit LDS address space).
__device__ inline uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// A wave-uniform value or resource forced into scalar registers (free when
// the compiler already keeps it there), as the "s" operands below require.
__device__ inline uint32_t sreg(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline u32x4 sreg(const u32x4 &r) {
  return (u32x4){sreg(r.x), sreg(r.y), sreg(r.z), sreg(r.w)};
}

// Wait states inside the assembly blocks below.  A VALU instruction that
// writes an SGPR (v_readfirstlane, or v_readlane when the compiler reloads a
// spilled SGPR) needs five wait states before a vector-memory instruction
// reads that SGPR as its resource or scalar offset (the gfx9 family's
// manually inserted wait states).  The compiler counts them for the
// vector-memory instructions it emits, but never for those inside inline
// assembly, and it may put such a write directly before the block: a store
// of the dense epilogue then used a stale scalar row offset whenever its
// SGPR had just been reloaded from a spill, writing rows of D to the wrong
// place in the transposed tensor-wise kernels of one build.  So every block
// issues at least five wait states before its memory instruction.
//
// lds: LDS byte address of lane 0's destination, uniform; IMM is added to
// it inside the instruction sequence so that call sites that differ only by
// a constant share one base register.  The buffer range check covers the
// vector offset only, never the scalar offset soff: soff may only carry a
// part of the offset that keeps every lane inside the resource.
template <int BYTES, int IMM = 0>
__device__ inline void dma_asm(uint32_t lds, const u32x4 &r, uint32_t voff, uint32_t soff) {
  static_assert(BYTES == 4 || BYTES == 16, "DMA width");
  if constexpr (BYTES == 16)
    asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 3\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(sreg(lds)), "v"(voff), "s"(sreg(r)), "s"(sreg(soff)), "i"(IMM) : "memory", "m0", "scc");
  else
    asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 3\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 ::"s"(sreg(lds)), "v"(voff), "s"(sreg(r)), "s"(sreg(soff)), "i"(IMM) : "memory", "m0", "scc");
}

// The same DMA with the whole source offset, voff + add (add uniform), in
// the vector offset, so that the range check sees all of it: lanes whose
// bytes lie past the resource's end read zeros and touch no memory.  The sum
// is formed inside the block (a temporary VGPR) so that the compiler does not
// precompute and keep every DMA's offset live.
template <int BYTES, int IMM = 0>
__device__ inline void dma_asm_v(uint32_t lds, const u32x4 &r, uint32_t voff, uint32_t add) {
  static_assert(BYTES == 4 || BYTES == 16, "DMA width");
  uint32_t t;
  if constexpr (BYTES == 16)
    asm volatile("s_add_u32 m0, %1, %5\n\tv_add_u32 %0, %4, %2\n\ts_nop 2\n\tbuffer_load_dwordx4 %0, %3, 0 offen lds"
                 : "=&v"(t) : "s"(sreg(lds)), "v"(voff), "s"(sreg(r)), "s"(sreg(add)), "i"(IMM) : "memory", "m0", "scc");
  else
    asm volatile("s_add_u32 m0, %1, %5\n\tv_add_u32 %0, %4, %2\n\ts_nop 2\n\tbuffer_load_dword %0, %3, 0 offen lds"
                 : "=&v"(t) : "s"(sreg(lds)), "v"(voff), "s"(sreg(r)), "s"(sreg(add)), "i"(IMM) : "memory", "m0", "scc");
}

// A 16-byte buffer store (D[voff + soff] = v) with wait states on both
// sides in one assembly block.  Before it: five, for an SGPR operand just
// written by a VALU instruction (see above).  After it: three, because the
// store reads its data VGPRs after it issues and a VALU write of those VGPRs
// in the next two cycles corrupts what is stored; the compiler's hazard
// checks assume no such hazard when soffset is an SGPR, which does not hold
// on gfx950 (seen as a wrong last dword in lanes 12-15 of each row of 16
// lanes).
__device__ inline void store16_asm(const v4i &v, const u32x4 &r, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_store_dwordx4 %0, %1, %2, %3 offen\n\ts_nop 2"
               ::"v"(v), "v"(voff), "s"(sreg(r)), "s"(sreg(soff)) : "memory");
}

// Compile-time loop: f(std::integral_constant<int, J>) for J in [B, E).
template <int B, int E, class F>
__device__ inline void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
#pragma clang diagnostic pop

__device__ inline uint32_t buf_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
}

// LDS accesses cast the generic pointer straight to the LDS address space
// (an address-space cast, not a round trip through an integer) so that
// alias information of the pointer survives.
__device__ inline v4i lds_read16(const void *p) {
  return *(const lds_v4i *)p;
}

__device__ inline v2i lds_read_tr8(const void *p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)p);
}

// ds_read_b64_tr_b4: each group of 16 lanes reads 8 bytes per lane (16
// nibbles) and receives the 16 x 16 nibble transpose: nibble j of lane i's
// result is nibble i of what lane j of its group read.
__device__ inline v2i lds_read_tr4(const void *p) {
  return __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_v2i *)p);
}

// D += sum over a 16x16x128 block: first operand rows = output rows.
template <int FX, int FY>
__device__ inline v4f mfma_scaled(const v8i &x, const v8i &y, const v4f &c, int sx, int sy) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, FX, FY, 0, sx, 0, sy);
}

// D += the 16x16x64 BF16 block held as an 8-bit operand fragment holds a
// 128-byte K chunk: lo half (K elements 8q .. 8q + 7 of a row, q = lane / 16)
// and hi half (32 + 8q ..) feed two 16x16x32 BF16 matrix-core instructions
// in K order.  First operand rows = output rows, as mfma_scaled.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
__device__ inline v4f mfma_bf16_x2(const v8i &x, const v8i &y, const v4f &c) {
  const bf16x8_t xl = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x, x, 0, 1, 2, 3));
  const bf16x8_t yl = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(y, y, 0, 1, 2, 3));
  const bf16x8_t xh = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x, x, 4, 5, 6, 7));
  const bf16x8_t yh = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(y, y, 4, 5, 6, 7));
  const v4f r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, yl, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, yh, r, 0, 0, 0);
}

// Two FP32 values -> packed BF16 (lo in bits 0-15), rounded to nearest
// even: one v_cvt_pk_bf16_f32 on gfx950 (the compiler's lowering of the
// vector conversion).  A NaN stays a NaN (its payload is not specified).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Epilogue activations (after the bias, on the FP32 result).
enum : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2, ACT_SILU = 3 };

// Logistic function 1 / (1 + e^-y) from the hardware base-2 exponential and
// reciprocal (each within about an ulp of FP32); saturates to 0 and 1.
__device__ inline float logistic_f32(float y) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * 1.4426950408889634f));
}

// GELU in its tanh form, z/2 (1 + tanh(u)) with u = sqrt(2/pi) (z +
// 0.044715 z^3), written as z * logistic(2u) (the two are equal since
// (1 + tanh(u)) / 2 = 1 / (1 + e^-2u)); SiLU z * logistic(z).
__device__ inline float activate(int act, float z) {
  if (act == ACT_RELU) return fmaxf(z, 0.0f);
  if (act == ACT_GELU_TANH) {
    const float u = 0.7978845608028654f * fmaf(0.044715f * z, z * z, z);
    return z * logistic_f32(2.0f * u);
  }
  if (act == ACT_SILU) return z * logistic_f32(z);
  return z;
}

__device__ inline uint32_t lds_load_u32(const void *p) { return *(const lds_u32_t *)p; }

}  // namespace mxg
