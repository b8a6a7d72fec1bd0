// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, MFMA wrappers, LDS transpose reads and the packed kernel
// argument block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_params.h"

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

#define PA_LDS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;   // log2(e): natural-log logits to exp2 units

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two float32 -> packed bf16x2 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 h = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
  __bf16 h = (__bf16)a;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposed 4 x b16 LDS read (gfx950 ds_read_b64_tr_b16).  Within every
// 16-lane group, lane i receives, as element e, the 16-bit word (i % 4) at the
// address supplied by lane 4*e + i/4 of the same group.  A group whose lanes
// point at rows r..r+3 (4 lanes per row, 4 consecutive columns each) thus
// returns column i of those 4 rows to lane i.
__device__ __forceinline__ u32x2 lds_read_tr16(const PA_LDS char* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Quantized cache codes -> bf16, exactly (|int8| <= 127 and every float8
// E4M3 value fit bf16's 8 significant bits).  Byte i of word w is code i.
enum KvCode : int { KV_BF16 = 0, KV_INT8 = 1, KV_FP8 = 2 };

__device__ __forceinline__ void i8x4_to_f32(uint32_t w, float (&f)[4]) {
  const uint32_t u = w ^ 0x80808080u;            // signed -> biased unsigned bytes
  f[0] = (float)(u & 0xffu) - 128.f;
  f[1] = (float)((u >> 8) & 0xffu) - 128.f;
  f[2] = (float)((u >> 16) & 0xffu) - 128.f;
  f[3] = (float)(u >> 24) - 128.f;
}
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float (&f)[4]) {
  // gfx950 converts OCP E4M3 (the float8_e4m3fn format) in hardware
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}
template <int KQ>
__device__ __forceinline__ void codes4_to_f32(uint32_t w, float (&f)[4]) {
  if constexpr (KQ == KV_INT8) i8x4_to_f32(w, f);
  else fp8x4_to_f32(w, f);
}
// 4 int8 codes c -> 4 bf16 holding c + 128 (0..255, exact): one conversion
// per value; the kernels subtract 128 times the operand sum afterwards.
__device__ __forceinline__ u32x2 i8x4_to_bf16_biased(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  return u32x2{pack_bf16x2((float)(u & 0xffu), (float)((u >> 8) & 0xffu)),
               pack_bf16x2((float)((u >> 16) & 0xffu), (float)(u >> 24))};
}

// 4 codes -> 4 bf16 (two packed words).  Float8 E4M3 goes straight to bf16,
// two codes per instruction (gfx950's scaled conversion with scale 1; every
// E4M3 value is a bf16 value, so it is exact).
template <int KQ>
__device__ __forceinline__ u32x2 codes4_to_bf16(uint32_t w) {
  if constexpr (KQ == KV_FP8) {
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  } else {
    float f[4];
    codes4_to_f32<KQ>(w, f);
    return u32x2{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
  }
}

// Cross-lane helpers over the 64-lane wave.
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  int lane = __lane_id();
  int src = lane ^ mask;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// Reductions across the two 32-lane halves of a wave (lane i with lane i^32)
// on the gfx950 half swap, which stays in the VALU (no LDS round trip).  The
// swap returns, in some order, the lane's own value and its partner's.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions across lanes i and i ^ 16 on the gfx950 row-pair swap (no LDS
// round trip); the swap returns, in some order, the lane's own value and
// its partner's.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Page id of logical page j of sequence b, clamped into the pool so a bad
// table entry can never address memory outside it.
__device__ __forceinline__ int page_of(const AttnParams& p, int b, int j) {
  int pg = p.block_tables[(int64_t)b * p.table_width + j];
  return clampi(pg, 0, p.num_pages - 1);
}

}  // namespace pa
