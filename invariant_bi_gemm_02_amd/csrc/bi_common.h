// bi_common.h -- device helpers shared by the HIP kernels of libbi.so.
// gfx950 (CDNA4) only: wave64, v_mfma_f32_16x16x32_bf16, ds_read_b64_tr_b16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define BI_LDS __attribute__((address_space(3)))

// bf16 bits -> fp32: exact (bf16 is the top half of binary32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u) return (u >> 16) | 0x0040u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// One matrix-core op: c += a(16x32) . b(32x16), bf16 in, fp32 accumulate.
// Operand layout on gfx950, lane l of the wave:
//   a: row l%16 of A, k = (l/16)*8 .. +7;   b: column l%16 of B, same k;
//   c: column l%16 of C, rows (l/16)*4 .. +3.
__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// acc + a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs (v_dot2_f32_bf16).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// LDS transpose read of 16-bit data.  Within each group of 16 lanes, lane
// 4r + c passes the address of 4 consecutive elements (row r, columns
// 4c..4c+3) of a 4x16 block; afterwards lane i of the group holds column i
// of the block, rows 0..3.
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* lds_addr) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BI_LDS i16x4_t*)(lds_addr));
  return __builtin_bit_cast(u32x2_t, v);
}

// The same read from a 32-bit LDS byte address (no generic-pointer cast).
__device__ __forceinline__ u32x2_t lds_read_tr16_at(uint32_t lds_byte_addr) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BI_LDS i16x4_t*)(uintptr_t)lds_byte_addr);
  return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ u32x4_t ldg128(const void* p) { return *(const u32x4_t*)p; }

// A load of data read once (weights at decode sizes, a K/V page, segment
// sums): the non-temporal hint (`nt`) streams it past the caches' normal
// replacement, which lets HBM deliver about 10% more to a streaming reader
// (a plain read of 1 GiB: 6.2 -> 6.8 TB/s).  Same value as ldg128.
__device__ __forceinline__ u32x4_t ldg128_nt(const void* p) {
  return __builtin_nontemporal_load((const u32x4_t*)p);
}

// Buffer resource over [base, base + bytes): raw (unswizzled) addressing with
// a 32-bit byte offset; reads at offsets >= bytes return zero in hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4_t bufld128(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
// The same load with the non-temporal hint (cache-policy bit 1, `nt` on
// gfx950), for data read once.
__device__ __forceinline__ u32x4_t bufld128_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}
__device__ __forceinline__ void stg128(void* p, const u32x4_t& v) { *(u32x4_t*)p = v; }

// Direct-to-LDS load: every lane fetches 16 bytes at byte offset `off` of the
// buffer; lane i's bytes land at lds_base + 16 i.  Reads past the end of the
// buffer deposit zeros.  Completion is counted by vmcnt, not by any register.
// Raw buffer resource as four dwords (base, stride 0, byte size, flags), for
// inline assembly operands.  Offsets at or past `bytes` read as zero.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return i32x4_t{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// Direct-to-LDS load of 16 bytes per lane: lane i's 16 bytes from byte offset
// voff land at LDS byte address lds_addr + 16 i (lds_addr wave-uniform).
// Issued from inline assembly so that the compiler's counter tracking does
// not see it: the caller waits (s_waitcnt vmcnt) before the data is read.
// M0, which the instruction takes the LDS address from, is restored.
__device__ __forceinline__ void lds_dma16(i32x4_t rsrc, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_addr)
      : "memory");
}

// The same load with a scalar byte offset added to voff (the buffer's range
// check applies to voff + soff): a per-stage advance carried in an SGPR
// leaves the per-lane offsets untouched.
__device__ __forceinline__ void lds_dma16_so(i32x4_t rsrc, uint32_t voff, uint32_t soff,
                                             uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr)
      : "memory");
}

}  // namespace bi
