// bf16 matrix-core (MFMA) helpers for gfx950, wave64.
//
// v_mfma_f32_32x32x16_bf16 lane layout (checked on the device):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) + 0..7
//   B (16 x 32): lane l holds col l%32, k = 8*(l/32) + 0..7
//   C (32 x 32): lane l, element v holds row 8*(v/4) + 4*(l/32) + v%4, col l%32
// The attention-style kernels compute transposed products (S^T = K Q^T) so that the
// softmax over keys runs along rows of the accumulator, i.e. inside one lane and its
// partner lane l^32. The accumulator of one 32-row tile, read as eight consecutive
// elements 8s..8s+7, is directly the B operand of the next product over those rows
// for k-step s when the A operand lists its k entries as rows
//   16s + 4*(l/32) + {0,1,2,3}  and  16s + 8 + 4*(l/32) + {0,1,2,3}
// of the 32-row tile (a fixed permutation of the k index, which a sum does not see).
//
// ds_read_b64_tr_b16 (checked on the device): within each group of 16 lanes, lane
// 4i + r supplies the address of four consecutive 16-bit elements (row i, columns
// 4r..4r+3 of a 4 x 16 block); lane j of the group receives column j of that block,
// rows 0..3. So an operand whose k index runs down the rows of a row-major LDS tile
// loads without any transposition: lane l of the wave gives row
// kbase + 8*(l/32) + (l%16)/4 (+4 for the second read), column cbase + 16*((l/16)%2)
// + 4*(l%4), and receives column cbase + l%32, rows kbase + 8*(l/32) + 0..3 (4..7).
#pragma once

#include "muse_common.hpp"

namespace muse {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) unsigned short u16x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned short u16x4_t;

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Four 16-bit elements through the LDS transpose read (address 8-byte aligned).
__device__ __forceinline__ u16x4_t lds_read_tr16(const uint16_t* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u16x4_t, r);
}

// One k-major MFMA operand (8 k values of column cbase + l%32, k = kbase + 8*(l/32) + 0..7)
// from a row-major LDS tile with row stride `ld` elements.
__device__ __forceinline__ bf16x8_t lds_operand_tr(const uint16_t* tile, int ld, int kbase, int cbase, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const uint16_t* p = tile + (kbase + 8 * (g >> 1) + (s >> 2)) * ld + cbase + 16 * (g & 1) + 4 * (s & 3);
  const u16x4_t r0 = lds_read_tr16(p);
  const u16x4_t r1 = lds_read_tr16(p + 4 * ld);
  const u16x8_t u = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(bf16x8_t, u);
}

// The same with the k order of an accumulator reused as B operand: lane l receives rows
// kbase + 4*(l/32) + 0..3 and kbase + 8 + 4*(l/32) + 0..3 of column cbase + l%32, i.e. the
// rows that accumulator elements 8s..8s+7 of a 32-row tile hold for kbase = 16 s.
__device__ __forceinline__ bf16x8_t lds_operand_tr_acc(const uint16_t* tile, int ld, int kbase, int cbase, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const uint16_t* p = tile + (kbase + 4 * (g >> 1) + (s >> 2)) * ld + cbase + 16 * (g & 1) + 4 * (s & 3);
  const u16x4_t r0 = lds_read_tr16(p);
  const u16x4_t r1 = lds_read_tr16(p + 8 * ld);
  const u16x8_t u = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u16x8_t& u) { return __builtin_bit_cast(bf16x8_t, u); }

// Eight fp32 values rounded to bf16 (nearest even).
__device__ __forceinline__ bf16x8_t pack_bf16x8(const float* x) {
  u16x8_t u;
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = f32_to_bf16_bits(x[i]);
  return as_bf16x8(u);
}

// hi = bf16(x), lo = bf16(x - hi): x == hi + lo up to 2^-16 relative.
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8_t& hi, bf16x8_t& lo) {
  u16x8_t h, l;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = f32_to_bf16_bits(x[i]);
    l[i] = f32_to_bf16_bits(x[i] - bf16_to_f32(h[i]));
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace muse
