// Device-side helpers shared by the gfx950 attention kernels: operand vector
// types, the MFMA forms used, and 16-bit float packing with round-to-nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_lds.hpp"
#include "fa_sched.hpp"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type tags.  Tensors are passed around as raw 16-bit words; the tag
// selects the MFMA form and the float<->16-bit conversions.
struct bf16_t {};
struct f16_t {};

template <typename T> struct Ops;

template <> struct Ops<bf16_t> {
  // D(32x32) += A(32x16) * B(16x32); one 16-byte operand per lane.
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // D(16x16) += A(16x32) * B(32x16).
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // D(16x16) += A(16x16) * B(16x16); 4 elements of 16 bits per lane.
  static __device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  // Two floats -> two bf16 (RNE) in one dword, `lo` in the low half.
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
};

template <> struct Ops<f16_t> {
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

#define FA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))
#define FA_GLOBAL(T, p) ((__attribute__((address_space(1))) T*)(p))

// s_waitcnt immediate that waits until at most n (< 64) of this wave's
// vector-memory operations are outstanding (vmcnt is split over bits 3:0 and
// 15:14; expcnt and lgkmcnt are left at their maxima).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Asynchronous 16-byte HBM -> LDS copy (buffer_load_dwordx4 ... lds) from a
// wave-uniform base plus a 32-bit per-lane byte offset.  `lds` must be the
// same for every lane of the wave: lane l's 16 bytes land at lds + 16*l.  The
// buffer form, not the global one (global_load_lds_dwordx4): the compiler
// treats the global form as a FLAT access that may touch LDS, so while one
// is in flight every wait for an LDS operand read drains all of them
// (lgkmcnt(0)); the buffer form counts on vmcnt alone and reads issued ahead
// keep exact partial waits.
// Descriptor: base, no stride, no range limit, 32-bit data format.  A base
// the compiler cannot prove wave-uniform makes it loop over the base's
// distinct values, so callers pass bases computed from uniform values only.
__device__ __forceinline__ void load_lds16_buf(const void* base, uint32_t off_bytes, void* lds) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, FA_LDS(void, lds), 16, off_bytes, 0, 0, 0);
}

// A pointer the caller knows to be wave-uniform, taken from the first active
// lane so that the compiler holds it in scalar registers.
template <typename P> __device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  return reinterpret_cast<P*>((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
                              ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32));
}

// Wait until this wave's vector-memory loads (including LDS-direct ones) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); }

// ds_read_b64_tr_b16.  Within each group of 16 lanes, lane i receives element
// (i % 4) of the 8-byte chunk addressed by lane 4k + i/4, for k = 0..3.  With
// lane j of the group pointing at row (r0 + j/4), columns c0 + 4*(j%4) .. +3
// of a row-major 16-bit matrix, lane i gets column c0 + i of rows r0..r0+3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(i16x4, p));
  return __builtin_bit_cast(u32x2, v);
}

// v_permlane32_swap(x, x) gives (x of lane l%32, x of lane l%32 + 32) in every
// lane, so a reduction across the two wave halves is one swap and one op.
__device__ __forceinline__ float max_halves(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Value held by lane (lane ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }
__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16); }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace fa
