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

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace kvs
