// Device helpers shared by the gfx950 kernels of libwaveprune.
#pragma once

#include "wp_internal.h"

namespace wp {

// dword 3 of a raw (untyped, stride 0) buffer resource on gfx9-family parts
constexpr int kBufferFlags = 0x00020000;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// The LDS address-space casts live in device-only helpers: the kernel body
// must stay valid for the host compilation pass that emits its launch stub.
// 16 bytes per lane from a raw buffer straight into LDS at dst + 16*lane.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, void* dst, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voffset, 0, 0, 0);
}
// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i % 4
// of the 4 x 16-bit values addressed by lanes 4e + i / 4, e = 0..3.
__device__ inline u32x2 read_tr16(const void* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

// LDS byte address of a pointer into __shared__ memory
__device__ inline unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)((const __attribute__((address_space(3))) void*)p);
}

// The two K operands (key blocks 0 and 1) of one S^T step, complete on
// return.  Written as one asm block with its own wait so that the compiler
// keeps it where it is placed (after the previous step's MFMAs) instead of
// sinking the reads next to their first use.
template <int OFF>
__device__ inline void k_reads(u32x4& a, u32x4& b, unsigned addr) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %2 offset:%3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b)
      : "v"(addr), "n"(OFF)
      : "memory");
}

__device__ inline f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (nearest even), one v_cvt_pk_bf16_f32
__device__ inline unsigned int pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// A raw buffer resource for [p, p + bytes) held in scalar registers: the
// base and size are wave-uniform by construction, readfirstlane makes that
// explicit so loads through it need no per-lane waterfall loop.
__device__ inline __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, 0, __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

// Combine x of lanes l and l ^ 32 (the two halves that hold one query
// column) with v_permlane32_swap, no LDS round trip.  Swapping rows 2-3 of
// (x) with rows 0-1 of (x) leaves every lane with x_lo in one result and
// x_hi in the other, so max / sum of the pair is the same in both halves.
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A 16-byte MFMA operand with the 4-byte words (dim pairs) for which
// keep(w) fails set to zero.
template <typename F>
__device__ inline u32x4 keep_words(const u32x4& x, F keep) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) r[w] = keep(w) ? x[w] : 0u;
  return r;
}

// Row (key) of register r of a 32x32 MFMA output block for lane half hh.
__device__ inline int out_row(int r, int hh) { return ((r >> 2) << 3) + (hh << 2) + (r & 3); }

}  // namespace wp
