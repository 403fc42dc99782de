// Tile helpers shared by the MFMA attention kernels (dense prefill, adjacent-query dedup).
//
// 32x32 MFMA output layout: lane l holds column l%32 and rows 8(i/4) + 4(l/32) + i%4, i<16.
// S^T = K Q^T: A row rr of a 32-key block loads key kperm(rr), so that per lane half the 8
// registers used by one PV k-step hold 8 consecutive keys.  The V^T operand of O^T += V^T P^T
// (fp16 P x fp16 V) comes straight from the natural [key][dim] V tile in LDS through
// ds_read_b64_tr_b16: inside each 16-lane group, lane j receives element j%4 of the 4-element
// rows fetched by lanes j/4, j/4+4, j/4+8 and j/4+12, so lanes that fetch (key k0 + i/4,
// dims d0 + 4(i%4)..+3) end up with keys k0..k0+3 of dim d0 + j.
#pragma once
#include "common.h"

namespace dsa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_f16_16x16x32(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16_32x32x16(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 8 fp32 -> 8 fp16 (round to nearest even), packed as 4 dwords.
__device__ __forceinline__ i32x4 pack_f16x8(const float* p) {
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)p[i];
  return __builtin_bit_cast(i32x4, h);
}

__device__ __forceinline__ uint16_t bf16_lane(const i32x4& v, int e) {
  const uint32_t w = uint32_t(v[e >> 1]);
  return uint16_t((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}

__device__ __forceinline__ int kperm(int rr) {
  const int a = rr >> 3, hh = (rr >> 2) & 1, bb = rr & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + bb;
}

constexpr int kKvRowB = 288;             // bytes per K/V row in LDS (256 + 32 pad)
constexpr int kKvTileB = 64 * kKvRowB;   // one 64-key tile

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<uint8_t*>(p)));
}

// 16-byte unit swizzle inside a K/V row: flips unit bit 0 with key bit 3 (removes the 2-way
// bank conflict between keys k and k+8 in the K-operand reads).
__device__ __forceinline__ int kv_off(int key, int byte) { return key * kKvRowB + (byte ^ (((key >> 3) & 1) << 4)); }


}  // namespace dsa
