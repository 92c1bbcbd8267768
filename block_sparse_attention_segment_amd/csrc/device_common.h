// Device-side helpers shared by the gfx950 kernels: vector types, bf16 packing, the
// 32x32x16 bf16 MFMA and cross-half wave exchange.
//
// MFMA v_mfma_f32_32x32x16_bf16 lane layout (checked on the device): with l the lane,
//   A (32 x 16, M x K): lane l holds A[l % 32][8 * (l / 32) + t], t = 0..7
//   B (16 x 32, K x N): lane l holds B[8 * (l / 32) + t][l % 32]
//   D (32 x 32):        lane l, register r holds D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace br {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Round two floats to bf16 (nearest even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane l ^ 32 (the other half of the wave), via v_permlane32_swap.
__device__ __forceinline__ float other_half(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // r[0] is the lower half's value and r[1] the upper half's, in every lane.
  const bool upper = (threadIdx.x & 32) != 0;
  return __uint_as_float(upper ? r[0] : r[1]);
}

__device__ __forceinline__ float max_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ u32x4_t load16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element (i % 4) of the four
// 16-bit values at the address of lane 4 j + i / 4, as its element j (j = 0..3).  Reading a
// row-major [key][d] tile with lane 4 j + q pointing at (key0 + j, d0 + 4 q) therefore gives
// lane i the four keys key0..key0+3 of column d0 + i: a transposed fragment.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));  // generic -> LDS address
  return __builtin_bit_cast(u32x2_t, v);
}

// Raw buffer resources (gfx9-family descriptor, 32-bit elements, no stride).  A buffer load whose
// byte offset is at or beyond `bytes` returns zeros and such a store is dropped, so tile edges need
// no branches.  `bytes` must fit in 31 bits; callers build one resource per tile or row block.
constexpr int kBufferDword3 = 0x00020000;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferDword3);
}
__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, uint32_t byte_offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0);
}
__device__ __forceinline__ void buf_store8(u32x2_t v, rsrc_t r, uint32_t byte_offset) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_offset, 0, 0);
}
__device__ __forceinline__ void buf_store16(u32x4_t v, rsrc_t r, uint32_t byte_offset) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_offset, 0, 0);
}
// The same with the non-temporal hint (cache policy bit 1, "nt" on gfx950), for whole-line writes
// that are not read again soon: the L2 then keeps the lines that are re-read in preference.
__device__ __forceinline__ void buf_store16_nt(u32x4_t v, rsrc_t r, uint32_t byte_offset) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_offset, 0, 2);
}
// Rotary embedding of packed bf16 pairs, fp32 arithmetic, one rounding to bf16 (shared by the
// rotation kernel and the attention kernel's in-register rotation of Q, so both round alike).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
// Split layout: x0 holds the first entries of pairs 0..7 (two per dword), x1 the second entries.
__device__ __forceinline__ void rope_rotate_split8(u32x4_t& x0, u32x4_t& x1, const float* cs, const float* sn) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a0 = bf16_lo(x0[i]), a1 = bf16_hi(x0[i]), b0 = bf16_lo(x1[i]), b1 = bf16_hi(x1[i]);
    const int j = 2 * i;
    x0[i] = pack_bf16x2(fmaf(a0, cs[j], -b0 * sn[j]), fmaf(a1, cs[j + 1], -b1 * sn[j + 1]));
    x1[i] = pack_bf16x2(fmaf(a0, sn[j], b0 * cs[j]), fmaf(a1, sn[j + 1], b1 * cs[j + 1]));
  }
}
// Adjacent layout: dword i of x is pair i (first entry in the low half).
__device__ __forceinline__ void rope_rotate_adjacent4(u32x4_t& x, const float* cs, const float* sn) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = bf16_lo(x[i]), b = bf16_hi(x[i]);
    x[i] = pack_bf16x2(fmaf(a, cs[i], -b * sn[i]), fmaf(a, sn[i], b * cs[i]));
  }
}

// Direct-to-LDS buffer load (gfx950 buffer_load_dwordx4 ... lds): lane l's 16 bytes at
// soffset + byte_offset go to LDS byte address lds_addr + 16 l (lds_addr: wave-uniform, from
// lds_addr_of).  Loads whose soffset + byte_offset reaches the resource's size write zeros (the
// scalar offset counts in the range check: checked on gfx950).  Completion is tracked by the vector-memory
// counter only: the caller waits for it (s_waitcnt vmcnt) before anything reads that LDS.  The
// instruction is issued from inline assembly so that the compiler does not add its own
// conservative vector-memory waits before every later LDS read; it has no register result.
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, uint32_t lds_addr, uint32_t byte_offset,
                                               uint32_t soffset = 0) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_addr), "v"(byte_offset),
               "s"(r), "s"(soffset)
               : "memory", "m0");
}
// The same with the non-temporal hint, for data read once (query rows): the L2 then keeps the
// lines that are re-read (keys and values) in preference to these.
__device__ __forceinline__ void buf_load16_lds_nt(rsrc_t r, uint32_t lds_addr, uint32_t byte_offset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(lds_addr), "v"(byte_offset),
               "s"(r)
               : "memory", "m0");
}
// The same for 4 bytes per lane (buffer_load_dword ... lds): lane l's dword goes to lds_addr + 4 l.
__device__ __forceinline__ void buf_load4_lds(rsrc_t r, uint32_t lds_addr, uint32_t byte_offset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds_addr), "v"(byte_offset), "s"(r)
               : "memory", "m0");
}
// LDS byte address of a __shared__ object (for M0).
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  typedef __attribute__((address_space(3))) const void lds_void_t;
  return uint32_t(uintptr_t((lds_void_t*)p));
}
// a.x * b.x + a.y * b.y + c for two packed bf16 pairs, fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

}  // namespace br
