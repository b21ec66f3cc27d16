// Device-side primitives shared by the VDN kernels (gfx950 / CDNA4).
//
// Storage types: bf16 values live in memory as uint16_t; MFMA operands are
// clang vector types.  All accumulation is fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdn {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(bf16_t, b);
}

// Two floats -> packed pair of bf16 in one dword (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// 16-byte vector load/store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing LDS read of 16-bit data (ds_read_b64_tr_b16, gfx950).  Each
// lane names 8 bytes; within every group of 16 lanes the reads are
// redistributed so that lane i of the group receives element i % 4 of the
// reads of group lanes 4 e + i / 4, e = 0..3.  With group lane s pointing at
// row r0 + s / 4, columns c0 + 4 (s % 4) .. + 3 of a row-major 16-bit tile,
// lane i receives column c0 + i of rows r0 .. r0 + 3: four consecutive
// contraction slots of an MFMA operand read from a tile stored the other way
// round.  p must be an LDS address, 8-byte aligned.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const bf16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Raw buffer loads (gfx9 buffer descriptor: stride 0, num_records = bytes,
// word 3 = 0x00020000).  A 16-byte load whose range lies past num_records
// returns zeros, so tile loads need no bounds branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// Largest byte count a descriptor can cover starting at `base` of a tensor
// whose end is `end` (clamped to 2^31 - 16).
__device__ __forceinline__ uint32_t rsrc_bytes(const void* base, const void* end) {
  const long long n = (const char*)end - (const char*)base;
  return (uint32_t)(n < 0 ? 0 : (n > 0x7FFFFFF0ll ? 0x7FFFFFF0ll : n));
}

// v_mfma_f32_32x32x16_bf16.  Operand layout (wave64): lane l supplies row
// (l % 32) of A / column (l % 32) of B with 8 consecutive k-slots of its half
// (l / 32).  A and B use the same k-slot mapping, so any bijection of the 16
// contracted indices onto (half, slot) gives the same product.  Result: lane
// l holds column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4) for i in [0,16).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and B[l/32][l%32].
__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row of the 32x32 MFMA result held in accumulator register i by a lane of
// half g (= lane / 32).
__device__ __forceinline__ constexpr int mfma32_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Reductions over the lane pair (l, l ^ 32) with v_permlane32_swap.  The
// swap returns, in each lane, its own value and its partner's (in an order
// that depends on the half), so a symmetric op of the two is the pair result.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS accesses only: vector-memory loads in
// flight stay in flight across it (a full __syncthreads waits for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace vdn
