// Device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
// (1, 1) in bf16: the second operand of a two-element bf16 sum by dot product
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ bf16x8 ld16(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ void st16(bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }

// Raw buffer resource over [base, base + bytes): loads at byte offsets at or
// beyond `bytes` return zero.  Addresses are an SGPR base, an SGPR offset and
// a 32-bit VGPR offset, so a wave needs one VGPR per access stream.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}


// Same, with the nontemporal hint: for streams read once whose every load
// instruction covers whole 128-byte lines.
__device__ __forceinline__ bf16x8 buffer_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2));
}

// 16x16x32 bf16 MFMA: A 16x32 (lane l: row l%16, k 8*(l/16)..+7),
// B 32x16 (lane l: column l%16, same k), C 16x16 (lane l: rows 4*(l/16)+r,
// column l%16).
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA: A 32x16 (lane l: row l%32, k 8*(l/32)..+7),
// B 16x32 (lane l: column l%32, same k), C 32x32 (lane l, register r:
// row 8*(r/4) + 4*(l/32) + r%4, column l%32).
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even float -> bf16 of eight values.
__device__ __forceinline__ bf16x8 to_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)f[i];
  return r;
}

__device__ __forceinline__ float wave_max_xor(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}

// max / sum of x over lanes l and l ^ 32 (the two wave halves), with
// v_permlane32_swap: after it, one register holds the lower and the other
// the upper half's value in every lane.  Written as assembly: the compiler
// here takes the builtin's two results for one value.  The s_nop is the wait
// a VALU write of the operands needs before the permute reads them.
__device__ __forceinline__ void half_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// Same for lanes l and l ^ 16 (v_permlane16_swap exchanges the odd and
// even 16-lane rows).
__device__ __forceinline__ void row_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float row_swap_max(float x) {
  float a = x, b = x;
  row_swap(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float row_swap_sum(float x) {
  float a = x, b = x;
  row_swap(a, b);
  return a + b;
}
__device__ __forceinline__ float half_swap_max(float x) {
  float a = x, b = x;
  half_swap(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float half_swap_sum(float x) {
  float a = x, b = x;
  half_swap(a, b);
  return a + b;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

// LDS-direct buffer load: lane l's 16 bytes at voff + soff of the resource
// land at LDS byte (lds + 16 l) (one wave fills 1 KB).  Out-of-range reads
// give zeros.  Not tracked by the compiler's wait counting: the caller waits
// with vmcnt(0) before the data is read.  The compiler's hazard checks do not
// look inside assembly, so the block waits for itself: a write of M0 needs
// one wait state before an LDS-direct load uses it (s_nop 0).  A VALU write of
// an SGPR the load reads (v_readfirstlane, v_readlane reloading a spilled
// resource word) would need five: callers keep every SGPR operand, the LDS
// address included, computed by scalar instructions (a wave-uniform index via
// readfirstlane once, outside the loops), and the generated code is scanned
// for such writes.  With s_nop 4 in every load, the loads' issue cost was
// measured at 2-5 % of the prefill.
__device__ __forceinline__ void lds_direct_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff, void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(r), "s"(soff), "{m0}"(m0)
               : "memory");
}

// Transposed LDS read (ds_read_b64_tr_b16) at an 8-byte aligned LDS address.
// Within each 16-lane group, lane i names 4 consecutive 16-bit elements of
// row i/4 of a 4 x 16 block (columns 4*(i%4) .. +3); lane j receives column
// j of the block's 4 rows.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                        (__attribute__((address_space(3))) s16x4*)(p)));
}

}  // namespace moa
