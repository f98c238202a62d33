// cdna4.hpp -- small gfx950 (CDNA4) device helpers shared by the attention-JVP
// kernels: vector types, buffer-resource loads, matrix-core wrappers and
// cross-lane reductions.  Device code only; no host logic lives here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ajvp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Buffer resource over [base, base + bytes): loads at or past `bytes` return 0
// and stores there are dropped, so no index can reach memory outside the
// tensor the descriptor names.  Word 3 is the gfx9 raw buffer format (32-bit
// data, no swizzle, no stride).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
// Same, with the offset split into a per-lane part and a wave-uniform part
// (kept in a scalar register); the range check applies to their sum.
// The same with the non-temporal hint, for data read for the last time.
__device__ inline u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2));
}
__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t uniform_off) {
  return __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)lane_off, (int)uniform_off, 0));
}

__device__ inline float buf_load4f(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0));
}

// Stores at or past the descriptor's size are dropped by the hardware.
__device__ inline void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, 0);
}
__device__ inline void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)byte_off, 0, 0);
}
__device__ inline void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)byte_off, 0, 0);
}

__device__ inline u32x4 lds_load16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void lds_store16(char* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// 32x32 output tile, 16-deep contraction, fp32 accumulate.  Operand lane
// layout: lane l holds row/column (l % 32) and the eight contraction slots
// 8*(l/32) .. 8*(l/32)+7.  Result: lane l holds column (l % 32) of rows
// 8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
__device__ inline f32x16 mma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ inline f32x16 mma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Pack eight fp32 values into fp16 (round to nearest even).
__device__ inline u32x4 pack_f16x8(float a0, float a1, float a2, float a3,
                                   float a4, float a5, float a6, float a7) {
  f16x8 h;
  h[0] = (_Float16)a0; h[1] = (_Float16)a1; h[2] = (_Float16)a2; h[3] = (_Float16)a3;
  h[4] = (_Float16)a4; h[5] = (_Float16)a5; h[6] = (_Float16)a6; h[7] = (_Float16)a7;
  return __builtin_bit_cast(u32x4, h);
}

// Two fp32 values to one register of two fp16 (round to nearest even).
__device__ inline uint32_t pack_f16x2(float a, float b) {
  f16x2 h;
  h[0] = (_Float16)a;
  h[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, h);
}

// Eight fp16 values times the fp16 pair in m (both halves equal), rounded to
// nearest even (packed fp16 multiplies).  Note: every __builtin_bit_cast here
// takes a whole vector or a scalar value; applied to an element of an
// ext_vector_type variable (x[i] as an lvalue) this compiler reads element 0
// whatever i is, so an element is first copied to a scalar.
__device__ inline u32x4 mul_f16x8(u32x4 x, uint32_t m) {
  const f16x2 mm = __builtin_bit_cast(f16x2, m);
  const f16x8 s = {mm[0], mm[0], mm[0], mm[0], mm[0], mm[0], mm[0], mm[0]};
  return __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, x) * s);
}

// acc + h.x + h.y for a register of two fp16 (products with 1.0 are exact;
// the sum is formed in fp32).
__device__ inline float add_f16x2(uint32_t h, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), one, acc, false);
}

// Value held by lane (l ^ 32): the other half of a 64-wide wave.
__device__ inline float swap_halves(float x) { return __shfl_xor(x, 32); }

// max / sum of x over lanes l and l ^ 32, in every lane (the max propagates
// NaN).  v_permlane32_swap exchanges the upper half of its first operand with
// the lower half of its second; with both set to x the two results hold x of
// the lower and of the upper half respectively, in every lane (a vector-ALU
// op, no LDS traffic).
__device__ inline float halves_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__builtin_bit_cast(float, (unsigned)r[0]),
                                       __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ inline float halves_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ inline bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

}  // namespace ajvp
