// Device-side helpers shared by the HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Value held by lane (l ^ 32): V_PERMLANE32_SWAP exchanges the upper half of the
// first operand with the lower half of the second; swapping x with itself leaves
// {x[l], x[l+32]} in lanes l < 32 and {x[l-32], x[l]} in lanes l >= 32.
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(threadIdx.x & 32 ? r[0] : r[1]);
}

__device__ __forceinline__ float max_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two floats -> two bf16 (round to nearest even) in one dword: V_CVT_PK_BF16_F32.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
  return __uint_as_float((unsigned)b << 16);
}

// OCP E4M3 decoding with the gfx950 conversion instructions (exact for every
// code: E4M3 values are representable in both bf16 and fp32).

// Four E4M3 codes (one dword) -> four bf16 packed in two dwords.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(unsigned w) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Four E4M3 codes (one dword) -> four floats.
__device__ __forceinline__ f32x4 e4m3x4_to_f32x4(unsigned w) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Order-preserving map float -> uint32 (larger float, larger key; -0 < +0).
__device__ __forceinline__ unsigned float_key(float f) {
  unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// All-lane wave reductions without the LDS crossbar: DPP moves pair lanes inside
// each 16-lane row (quad_perm [1,0,3,2] and [2,3,0,1], then the 8- and 16-lane
// mirrors), V_PERMLANE16_SWAP pairs rows 0-1 and 2-3, V_PERMLANE32_SWAP the two
// halves.  Each swap of x with itself returns, in its two results, every lane's
// own value and its partner's, so combining them reduces the pair in all lanes.
// Every lane combines the same two partial values at every step (in one order or
// the other, which commutative operations do not see), so all lanes end with the
// same bits, and the fixed tree makes results reproducible run to run.
#define BSA_DPP(x, ctrl) __builtin_amdgcn_update_dpp((x), (x), (ctrl), 0xF, 0xF, false)

template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce(T x, Op op) {
  static_assert(sizeof(T) == 4, "32-bit lanes");
  auto bits = [](T v) { return __builtin_bit_cast(int, v); };
  auto val = [](int v) { return __builtin_bit_cast(T, v); };
  x = op(x, val(BSA_DPP(bits(x), 0xB1)));   // quad_perm [1,0,3,2]
  x = op(x, val(BSA_DPP(bits(x), 0x4E)));   // quad_perm [2,3,0,1]
  x = op(x, val(BSA_DPP(bits(x), 0x141)));  // row_half_mirror
  x = op(x, val(BSA_DPP(bits(x), 0x140)));  // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap((unsigned)bits(x), (unsigned)bits(x), false,
                                                    false);
  x = op(val((int)r16[0]), val((int)r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap((unsigned)bits(x), (unsigned)bits(x), false,
                                                    false);
  return op(val((int)r32[0]), val((int)r32[1]));
}

__device__ __forceinline__ float wave_sum(float x) {
  return wave_allreduce(x, [](float a, float b) { return a + b; });
}

__device__ __forceinline__ float wave_max(float x) {
  return wave_allreduce(x, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ int wave_sum_int(int x) {
  return wave_allreduce(x, [](int a, int b) { return a + b; });
}

__device__ __forceinline__ int wave_min_int(int x) {
  return wave_allreduce(x, [](int a, int b) { return a < b ? a : b; });
}

__device__ __forceinline__ unsigned wave_max_uint(unsigned x) {
  return wave_allreduce(x, [](unsigned a, unsigned b) { return a > b ? a : b; });
}

__device__ __forceinline__ unsigned wave_min_uint(unsigned x) {
  return wave_allreduce(x, [](unsigned a, unsigned b) { return a < b ? a : b; });
}

__device__ __forceinline__ unsigned long long ballot64(bool p) { return __ballot(p); }

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int l = lane_id();
  return l ? (~0ull >> (64 - l)) : 0ull;
}

}  // namespace bsa
