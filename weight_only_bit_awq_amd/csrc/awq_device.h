// Device-side helpers shared by the gfx950 kernels of this library.
//
// Code decode ("magic number" conversion): OR-ing a 4-bit code c into the
// low mantissa bits of fp16 1024.0 (0x6400) gives the exact fp16 value
// 1024 + c; OR-ing it into bits 4..7 of fp16 64.0 (0x5400), whose mantissa
// step is 1/16, gives 64 + c. In the device layout a word holds rows k0..k0+7
// in nibble positions 0,4 | 1,5 | 2,6 | 3,7 for row pairs (0,1) | (2,3) |
// (4,5) | (6,7), so four mask-and-or operations (one after an 8-bit shift)
// yield the eight rows as fp16 pairs carrying the offsets 1024 or 64.
// Subtracting (offset + z) in fp16 is exact (small integers), so
//   d = q - z          exactly, as fp16, and
//   w = d * s          is the exact product rounded once to fp16 (RNE),
// which is the dequantised weight bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Raw buffer resources: loads whose byte offset is at or beyond the
// resource's size return zero without touching memory, which gives
// branch-free masking of rows and columns outside the matrix. Offsets are
// 32-bit, so every buffer addressed this way is below 2 GiB (checked on the
// host). 0x00020000 is the descriptor word 3 of the gfx9 family.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Copy 16 (or 4) bytes per lane from the buffer at byte offset `off` into
// LDS at lds + 16 * lane (lds + 4 * lane); out-of-range offsets write zeros.
// The size must be a literal here: inside a template the host pass of the
// compiler rejects it.
__device__ __forceinline__ void load_to_lds16(rsrc_t r, char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void load_to_lds4(rsrc_t r, char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 4, off, 0, 0, 0);
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Packed fp16 constants -(1024 + z) and -(64 + z) for a zero point z (0..15),
// built from bit patterns: fp16(-1024 - z) = 0xE400 | z, fp16(-64 - z) = 0xD400 | z<<4.
struct ZeroConst {
  uint32_t c1024;
  uint32_t c64;
};

__device__ __forceinline__ ZeroConst zero_const(uint32_t z) {
  uint32_t zz = z | (z << 16);
  ZeroConst c;
  c.c1024 = 0xE400E400u | zz;
  c.c64 = 0xD400D400u | (zz << 4);
  return c;
}

// Eight rows (q - z) of one device word, exact, as fp16.
__device__ __forceinline__ h8 decode_diff(uint32_t w, ZeroConst c) {
  const uint32_t w8 = w >> 8;
  const h2 p0 = as_h2((w & 0x000F000Fu) | 0x64006400u) + as_h2(c.c1024);
  const h2 p1 = as_h2((w & 0x00F000F0u) | 0x54005400u) + as_h2(c.c64);
  const h2 p2 = as_h2((w8 & 0x000F000Fu) | 0x64006400u) + as_h2(c.c1024);
  const h2 p3 = as_h2((w8 & 0x00F000F0u) | 0x54005400u) + as_h2(c.c64);
  h8 r;
  r[0] = p0[0]; r[1] = p0[1];
  r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1];
  r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Eight dequantised rows fp16((q - z) * s) of one device word.
__device__ __forceinline__ h8 decode_weight(uint32_t w, ZeroConst c, h2 s2) {
  const uint32_t w8 = w >> 8;
  const h2 p0 = (as_h2((w & 0x000F000Fu) | 0x64006400u) + as_h2(c.c1024)) * s2;
  const h2 p1 = (as_h2((w & 0x00F000F0u) | 0x54005400u) + as_h2(c.c64)) * s2;
  const h2 p2 = (as_h2((w8 & 0x000F000Fu) | 0x64006400u) + as_h2(c.c1024)) * s2;
  const h2 p3 = (as_h2((w8 & 0x00F000F0u) | 0x54005400u) + as_h2(c.c64)) * s2;
  h8 r;
  r[0] = p0[0]; r[1] = p0[1];
  r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1];
  r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ h2 splat_h2(uint16_t bits) {
  return as_h2((uint32_t)bits | ((uint32_t)bits << 16));
}

// (a & m) | o with m and o held in VGPRs (see decode_consts): the compiler
// then selects one v_and_or_b32 (gfx9 VOP3 encodes no literal operands; with
// literal masks it emits a separate AND and OR).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) { return (a & m) | o; }

struct DecodeConsts {
  uint32_t m1, m2, o1, o2;  // 0x000F000F, 0x00F000F0, 0x64006400, 0x54005400 in VGPRs
};

__device__ __forceinline__ DecodeConsts decode_consts() {
  DecodeConsts k;
  k.m1 = 0x000F000Fu;
  k.m2 = 0x00F000F0u;
  k.o1 = 0x64006400u;
  k.o2 = 0x54005400u;
  // opaque to the optimiser: keeps the constants in VGPRs
  asm volatile("" : "+v"(k.m1), "+v"(k.m2), "+v"(k.o1), "+v"(k.o2));
  return k;
}

// Eight rows (q - z) of one device word, exact, as fp16.
__device__ __forceinline__ h8 decode_diff_vk(uint32_t w, ZeroConst c, const DecodeConsts& k) {
  const uint32_t w8 = w >> 8;
  const h2 p0 = as_h2(and_or(w, k.m1, k.o1)) + as_h2(c.c1024);
  const h2 p1 = as_h2(and_or(w, k.m2, k.o2)) + as_h2(c.c64);
  const h2 p2 = as_h2(and_or(w8, k.m1, k.o1)) + as_h2(c.c1024);
  const h2 p3 = as_h2(and_or(w8, k.m2, k.o2)) + as_h2(c.c64);
  h8 r;
  r[0] = p0[0]; r[1] = p0[1];
  r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1];
  r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Eight dequantised rows fp16((q - z) * s) of one device word.
__device__ __forceinline__ h8 decode_weight_vk(uint32_t w, ZeroConst c, h2 s2, const DecodeConsts& k) {
  const uint32_t w8 = w >> 8;
  const h2 p0 = (as_h2(and_or(w, k.m1, k.o1)) + as_h2(c.c1024)) * s2;
  const h2 p1 = (as_h2(and_or(w, k.m2, k.o2)) + as_h2(c.c64)) * s2;
  const h2 p2 = (as_h2(and_or(w8, k.m1, k.o1)) + as_h2(c.c1024)) * s2;
  const h2 p3 = (as_h2(and_or(w8, k.m2, k.o2)) + as_h2(c.c64)) * s2;
  h8 r;
  r[0] = p0[0]; r[1] = p0[1];
  r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1];
  r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Zero point of column n from packed zeros row (words of 8 nibbles along N).
__device__ __forceinline__ uint32_t zero_nibble(uint32_t word, int n) {
  return (word >> (4 * (n & 7))) & 0xFu;
}

// Map a linear workgroup id to a work id so that consecutive work ids run on
// the same XCD: the dispatcher places workgroup b on XCD b % 8. XCD x gets
// the contiguous work ids [x*q + min(x, r), ...) with q = nb / 8, r = nb % 8;
// the map is a bijection on [0, nb).
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int xcds = 8;
  const int x = b % xcds;
  const int q = nb / xcds;
  const int r = nb % xcds;
  return x * q + (x < r ? x : r) + b / xcds;
}

}  // namespace awq
