// Internal helpers shared by the gfx950 kernels of libgdla (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef __bf16 bf16;
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define GDLA_DEV __device__ __forceinline__

// f(std::integral_constant<int, i>) for i = B .. E-1, unrolled at compile time
template <int B, int E, class F>
GDLA_DEV void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// gfx950 matrix cores, bf16 inputs, fp32 accumulation.
//   32x32x16: A lane l supplies row l%32, k = 8*(l/32)+e (e = vector element);
//             B lane l supplies column l%32, the same k; D lane l holds
//             column l%32, rows 8*i + 4*(l/32) + j in element 4*i + j.
GDLA_DEV f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// The same shape with fp16 inputs (the same rate).
GDLA_DEV f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
//   16x16x32: A lane l supplies row l%16, k = 8*(l/16)+e; B column l%16;
//             D lane l holds column l%16, rows 4*(l/16) + j.
GDLA_DEV f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 bytes global -> LDS without registers: lane i of the wave writes LDS bytes
// [lds + 16 i, lds + 16 i + 16) (lds must be wave-uniform).  Completion is
// tracked by vmcnt.
__device__ __forceinline__ void g2lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// The same copy issued from inline assembly: the compiler does not know that it
// writes LDS, so it adds no waits for it before later LDS reads.  The caller
// orders it with explicit s_waitcnt vmcnt counts and barriers.  `lds` must be
// wave-uniform (it goes to M0); the instruction has no register results.
__device__ __forceinline__ void g2lds16_explicit(const void* src, void* lds) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(__attribute__((address_space(3))) char*)lds);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(m0v)
      : "memory", "m0");
}

// As g2lds16_explicit, for data read once: the non-temporal policy bit keeps
// the stream from displacing reused lines (on gfx950 a stream of such loads
// runs at about 7.2 TB/s against 5.8 TB/s without the bit).
__device__ __forceinline__ void g2lds16_stream(const void* src, void* lds) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(__attribute__((address_space(3))) char*)lds);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off nt"
      :
      : "v"(src), "s"(m0v)
      : "memory", "m0");
}

// g2lds16_stream of src + OFF bytes, with OFF in the instruction's offset
// field (saves a 64-bit address add per load; 0 <= OFF < 4096).  The
// instruction adds its offset to the LDS address too, so M0 gets lds - OFF.
template <int OFF>
__device__ __forceinline__ void g2lds16_stream_off(const void* src, void* lds) {
  static_assert(OFF >= 0 && OFF < 4096, "instruction offset is 13-bit signed");
  const unsigned m0v = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(__attribute__((address_space(3))) char*)lds - (unsigned)OFF);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off offset:%2 nt"
      :
      : "v"(src), "s"(m0v), "i"(OFF)
      : "memory", "m0");
}

GDLA_DEV float to_f32(bf16 v) { return (float)v; }
GDLA_DEV float to_f32(float v) { return v; }
template <class T> GDLA_DEV T from_f32(float v);
template <> GDLA_DEV float from_f32<float>(float v) { return v; }
template <> GDLA_DEV bf16 from_f32<bf16>(float v) { return (bf16)v; }   // round to nearest even
template <> GDLA_DEV f16 from_f32<f16>(float v) { return (f16)v; }     // round to nearest even

GDLA_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// sigmoid with the hardware reciprocal (1 ulp) instead of the correctly rounded
// division sequence: 1/(1 + e^-z) saturates to 0 and 1 through rcp(inf) = 0
GDLA_DEV float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

GDLA_DEV float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
GDLA_DEV float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__host__ __device__ static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
