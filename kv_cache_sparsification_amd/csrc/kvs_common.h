// Internal helpers shared by the libkvs HIP sources (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvs.h"

namespace kvs {

// ---------------------------------------------------------------- host-side status
int fail(int code, const char* fmt, ...);        // records the message, returns code
int launch_status(const char* what);             // KVS_OK or KVS_E_HIP after a launch
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int kBlock = KVS_BLOCK_SIZE;           // tokens per paged block
constexpr int kWave = 64;                        // CDNA wavefront width

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16, round to nearest even: gfx950 converts in hardware (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r[0] = static_cast<__bf16>(lo);
  r[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float wave_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// Lane l and lane l ^ 32 combined without LDS: v_permlane32_swap hands each lane the pair
// {own value, partner's value} (in either order), which suits commutative operations.
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return a > b ? a : b;
}
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Word 3 of a gfx9-family buffer descriptor: 32-bit data format (untyped loads are then valid)
// and raw addressing, so each load is range-checked against the descriptor's byte count and
// reads zero past it.
constexpr int kBufferFlags = 0x00020000;

// 16 bytes per lane from a buffer straight into LDS: lane i's bytes land at lds + 16 * i (the
// LDS address must be the same for the whole wavefront).  Callers must not depend on what
// out-of-range lanes leave in LDS.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}

// gfx950 transposing LDS read: within each group of 16 lanes, lane j supplies the address of 4
// consecutive 16-bit values (row j/4, values 4*(j%4) .. +3 of a 4 x 16 block) and receives
// column j of the block, i.e. the 4 values the group's addresses hold at position j.
__device__ __forceinline__ u32x2 ds_read_tr16_b64(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  return __builtin_bit_cast(u32x2, r);
}

// ---------------------------------------------------------------- 8-bit cache (OCP E4M3)
// gfx950's fp8 conversions use the OCP E4M3 encoding (bias 7, 3 mantissa bits, largest finite
// magnitude 448, no infinities) and round to nearest even; they do not saturate, so values
// are clamped to +-448 first (fmed3 keeps the sign of zero).
constexpr float kE4M3Max = 448.f;
constexpr float kTinyRow = 0x1p-112f;   // rows whose largest magnitude is below this are stored as zeros

// Per-row quantization parameters: the stored scale amax/448 and the multiplier 448/amax
// (each one float32 division); both zero for a row stored as zeros.
__device__ __forceinline__ void e4m3_row_params(float amax, float& scale, float& r) {
  const bool live = amax >= kTinyRow;
  scale = live ? amax / kE4M3Max : 0.f;
  r = live ? kE4M3Max / amax : 0.f;
}

// Four values times r to four codes (byte i = value i).  r == 0 (a zero row) gives code 0.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float r) {
  if (r == 0.f) return 0u;
  a = __builtin_amdgcn_fmed3f(a * r, kE4M3Max, -kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b * r, kE4M3Max, -kE4M3Max);
  c = __builtin_amdgcn_fmed3f(c * r, kE4M3Max, -kE4M3Max);
  d = __builtin_amdgcn_fmed3f(d * r, kE4M3Max, -kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Codes to bf16 (exact: every E4M3 value is a bf16 value) with gfx950's scaled conversion at
// scale 1: two codes per instruction, byte order kept (bytes 0, 1 with word_sel false).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t c, bool hi) {
  const bf16x2v r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ short4_t e4m3x4_to_bf16x4(uint32_t c) {
  return __builtin_bit_cast(short4_t, u32x2{e4m3x2_to_bf16x2(c, false), e4m3x2_to_bf16x2(c, true)});
}
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 c) {
  return __builtin_bit_cast(bf16x8, u32x4{e4m3x2_to_bf16x2(c[0], false), e4m3x2_to_bf16x2(c[0], true),
                                          e4m3x2_to_bf16x2(c[1], false), e4m3x2_to_bf16x2(c[1], true)});
}

// Eight bf16 (one 16-byte chunk) times r to eight codes.
__device__ __forceinline__ u32x2 e4m3x8_from_bf16(u32x4 v, float r) {
  u32x2 out;
  out[0] = e4m3x4(bf16_bits_to_f32(v[0] & 0xffffu), bf16_bits_to_f32(v[0] >> 16), bf16_bits_to_f32(v[1] & 0xffffu),
                  bf16_bits_to_f32(v[1] >> 16), r);
  out[1] = e4m3x4(bf16_bits_to_f32(v[2] & 0xffffu), bf16_bits_to_f32(v[2] >> 16), bf16_bits_to_f32(v[3] & 0xffffu),
                  bf16_bits_to_f32(v[3] >> 16), r);
  return out;
}

__device__ __forceinline__ float absmax_bf16x8(u32x4 v) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(bf16_bits_to_f32(v[i] & 0xffffu)));
    m = fmaxf(m, fabsf(bf16_bits_to_f32(v[i] >> 16)));
  }
  return m;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace kvs
