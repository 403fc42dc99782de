// Shared device helpers for the gfx950 DSA kernels (CDNA4: wave64, MFMA, 160 KiB LDS).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kDecodeKeysPerBlock = 256;   // cached keys per decode-indexer workgroup (one range slot each)
constexpr int kDecodeTopkBins = 2048;      // value bins per sequence of the decode top-k histogram
constexpr int kDecodeTopkChunk = 4096;     // scores per decode top-k chunk (one candidate list each)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Monotone map of an fp32 score to uint32 (larger score -> larger key).  -0.0 is folded
// into +0.0 so that equal scores always give equal keys.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact value of an OCP e4m3 ("fn") code (sign, 4 exponent bits with bias 7, 3 mantissa bits;
// exponent 0 is subnormal).  The NaN code is never produced by the inputs here.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = (e == 0) ? float(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -mag : mag;
}

// Reinterpret 4 dwords as 8 bf16 for the MFMA builtins.
__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 16x16x128 fp8(e4m3) x fp8(e4m3) -> fp32, no block scale (format selects 0/0 = e4m3).
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Sequence lookup: largest b with cu[b] <= t (cu non-decreasing, cu[0] = 0).
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int nseq, int64_t t) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Offset (in floats) of 16-row score block j of a sequence inside its score triangle:
// block j holds rows 16j..16j+15, each with a stride of 16(j+1) floats.
__device__ __forceinline__ int64_t score_block_offset(int64_t j) { return 128 * j * (j + 1); }

}  // namespace dsa
