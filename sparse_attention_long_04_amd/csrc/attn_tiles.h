// Tile helpers shared by the MFMA attention kernels (dense prefill, adjacent-query dedup, the
// backward), and the direct global -> LDS copies with their barriers.
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
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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

constexpr int kKvRowB = 256;             // bytes per K/V row in LDS
constexpr int kKvTileB = 64 * kKvRowB;   // one 64-key tile

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<uint8_t*>(p)));
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ s16x4 lds_tr16_l(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(const_cast<lds_u8*>(p)));
}

// 16-byte unit swizzle inside a K/V row: unit u of key r sits at u ^ (4 (r % 4) + (r / 4) % 4).
// Conflict-free for the 16-byte operand reads of 16 consecutive keys (rows kperm(0..15) are 16
// distinct keys mod 16) and for the transposed 8-byte reads (4 consecutive keys x 4 units).
__device__ __forceinline__ int kv_off(int key, int byte) {
  return key * kKvRowB + (byte ^ ((((key & 3) << 2) | ((key >> 2) & 3)) << 4));
}

// ---- direct global -> LDS copies

// 16 bytes per lane from global memory (base + off, base wave-uniform) to LDS address
// lds_addr + 16 * lane (lds_addr wave-uniform).  Issued from asm so that the compiler's own
// wait counting leaves it alone (for some LDS reads it would otherwise wait for every copy in
// flight); the kernels wait for these copies themselves (lds_sync_vm) before a stage is read.
// M0 (the copy's LDS address) is saved and restored around it; the copy reads M0 one wait state
// after it is written.
__device__ __forceinline__ void dn_copy16(const void* base, uint32_t off, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds_addr)
      : "memory");
}
// As dn_copy16 for lanes 0..15 only: 256 bytes to lds_addr .. lds_addr + 255.  The exec mask is
// narrowed and restored inside the asm, so the caller has no branch.
__device__ __forceinline__ void dn_copy16_lo16(const void* base, uint32_t off, uint32_t lds_addr) {
  uint32_t saved;
  uint64_t ex;
  asm volatile(
      "s_mov_b64 %1, exec\n\ts_mov_b64 exec, 0xffff\n\ts_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0\n\ts_mov_b64 exec, %1"
      : "=&s"(saved), "=&s"(ex)
      : "v"(off), "s"(base), "s"(lds_addr)
      : "memory");
}

// Workgroup barrier once at most VM of the wave's memory loads (in issue order: all but its
// VM newest) are still in flight and its LDS reads have returned (s_waitcnt vmcnt(VM)
// lgkmcnt(0); gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  The compiler
// fences keep LDS accesses on their side of the barrier.
template <int VM>
__device__ __forceinline__ void lds_sync_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0070);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// every copy of the wave has landed
__device__ __forceinline__ void dn_sync() { lds_sync_vm<0>(); }
// as lds_sync_vm without waiting for the wave's LDS reads (the compiler has already waited for
// every read whose value was used)
template <int VM>
__device__ __forceinline__ void lds_sync_vm_nolgkm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0F70);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int I>
using dn_ic = std::integral_constant<int, I>;

__device__ __forceinline__ i32x4 dn_ld128(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(p);
}


}  // namespace dsa
