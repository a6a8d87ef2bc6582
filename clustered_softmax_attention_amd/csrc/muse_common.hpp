// Shared device helpers of the MuSe HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace muse {

// bfloat16 stored as raw bits; arithmetic always happens in fp32.
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (the hardware conversion, v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
};

template <>
struct Elem<bf16> {
  static __device__ __forceinline__ float load(const bf16* p, size_t i) { return bf16_to_f32(p[i].bits); }
  static __device__ __forceinline__ void store(bf16* p, size_t i, float x) { p[i].bits = f32_to_bf16_bits(x); }
};

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Wave-wide reductions (64 lanes) through shuffles; every lane gets the result.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Opt-in per-kernel timing: while enabled, every launch is bracketed by a pair of HIP
// events recorded on its stream (see muse_prof_* in include/muse.h).
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t e0_;
  hipEvent_t e1_;
};

// Kernels that use more than 64 KiB of dynamic LDS must opt in (gfx950 has 160 KiB).
inline void allow_lds(const void* fn, size_t bytes) {
  if (bytes > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

}  // namespace muse
