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

// Cross-lane moves on the VALU (no LDS crossbar). Lane-order facts, checked on the
// device: DPP quad_perm(1,0,3,2) / (2,3,0,1) exchange lanes l^1 / l^2, row_half_mirror
// maps lane i of each 8-lane half-row to 7 - i, row_ror:8 exchanges l^8 inside a
// 16-lane row; permlane16_swap(x, x) leaves in its two results the values of rows
// {r, r^1} of lane l, and permlane32_swap(x, x) the values of lanes {l, l^32}.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

// permlane{16,32}_swap of x with itself. The second operand is passed through an empty
// asm statement so that the compiler keeps the two swapped registers apart (with one
// value for both operands it has been seen to feed the swap a stale register).
struct SwapPair {
  unsigned r0, r1;
};
__device__ __forceinline__ SwapPair self_swap32(unsigned u) {
  unsigned b = u;
  asm volatile("" : "+v"(b));
  const auto r = __builtin_amdgcn_permlane32_swap(u, b, false, false);
  return {r[0], r[1]};
}
__device__ __forceinline__ SwapPair self_swap16(unsigned u) {
  unsigned b = u;
  asm volatile("" : "+v"(b));
  const auto r = __builtin_amdgcn_permlane16_swap(u, b, false, false);
  return {r[0], r[1]};
}

// The value of lane l ^ 32.
__device__ __forceinline__ float xor32(float x) {
  const SwapPair r = self_swap32(__builtin_bit_cast(unsigned, x));
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r.r0 : r.r1);
}
__device__ __forceinline__ int xor32(int x) {
  const SwapPair r = self_swap32(static_cast<unsigned>(x));
  return static_cast<int>((threadIdx.x & 32) ? r.r0 : r.r1);
}

// Wave-wide reductions (64 lanes); every step pairs two lanes symmetrically, so all
// lanes compute the same operands in the same order and get bit-identical results.
template <typename Op>
__device__ __forceinline__ float wave_reduce(float x, Op op) {
  x = op(x, dpp_f32<0xB1>(x));   // l ^ 1
  x = op(x, dpp_f32<0x4E>(x));   // l ^ 2
  x = op(x, dpp_f32<0x141>(x));  // the other quad of the half-row
  x = op(x, dpp_f32<0x128>(x));  // l ^ 8
  {
    const SwapPair r = self_swap16(__builtin_bit_cast(unsigned, x));
    x = op(__builtin_bit_cast(float, r.r0), __builtin_bit_cast(float, r.r1));
  }
  {
    const SwapPair r = self_swap32(__builtin_bit_cast(unsigned, x));
    x = op(__builtin_bit_cast(float, r.r0), __builtin_bit_cast(float, r.r1));
  }
  return x;
}

// Workgroups go to the 8 XCDs round-robin by linear index. This maps a linear index to
// a logical one such that every XCD takes one contiguous range of the logical order, so
// that neighbouring work items (which read the same data) share that XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int id, int total) {
  constexpr int X = 8;
  const int q = total / X, r = total % X, x = id % X, k = id / X;
  return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// Max over each 32-lane half of the wave (both halves reduced independently).
__device__ __forceinline__ float half_wave_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x128>(x));
  const SwapPair r = self_swap16(__builtin_bit_cast(unsigned, x));
  return fmaxf(__builtin_bit_cast(float, r.r0), __builtin_bit_cast(float, r.r1));
}

__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, [](float p, float q) { return fmaxf(p, q); });
}

__device__ __forceinline__ float wave_sum(float x) {
  return wave_reduce(x, [](float p, float q) { return p + q; });
}

__device__ __forceinline__ int wave_sum_int(int x) {
  x += dpp_i32<0xB1>(x);
  x += dpp_i32<0x4E>(x);
  x += dpp_i32<0x141>(x);
  x += dpp_i32<0x128>(x);
  {
    const SwapPair r = self_swap16(static_cast<unsigned>(x));
    x = static_cast<int>(r.r0 + r.r1);
  }
  {
    const SwapPair r = self_swap32(static_cast<unsigned>(x));
    x = static_cast<int>(r.r0 + r.r1);
  }
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
