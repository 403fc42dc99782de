// Backward of the sparse GQA attention over the selected keys (Keye-VL-2.0 summary page, gsyq.cn,
// section 一: after the dense warm-up, the "sparse adaptation" stage unfreezes every parameter
// and trains the model in sparse mode, which needs the gradients of this attention).
//
// With P = softmax over s in S_t of scale q[t,h] . k[s,g], O = P V, an upstream gradient dO and
// D[t,h] = dO[t,h] . O[t,h]:
//     dS = P (dO . v[s] - D),  dq[t,h] = scale sum_s dS k[s],
//     dk[s,g] = scale sum_{(t,h): s in S_t} dS q[t,h],  dv[s,g] = sum_{(t,h): s in S_t} P dO[t,h].
// No float atomics anywhere, so results are bit-identical run to run:
//   bwd_delta_kernel    D = rowsum(dO * O), 16 lanes per (row, head).
//   dq: dedup_dq_kernel over the union of each 16-row block's selected keys (union_kernel):
//     the dedup attention tile loop with S = K Q^T and dP = V dO^T, the row masks,
//     P = 2^(S scale - lse), dS = P (dP - D), and dq^T += K^T dS^T.
//   dk, dv: every key needs the rows that selected it, in a fixed order.  sel_bitmap_kernel
//     builds, per 32-row block of a sequence, one 32-bit word per key position (bit r = row r of
//     the block selected the key), with LDS integer atomics only.  sparse_dkv_kernel then takes
//     128 keys x one KV head (4 waves x 32 keys as MFMA columns) and a slice of the rows,
//     streams tiles of 64 (row, head) vectors (8 rows x 8 heads for groups of 8) through LDS,
//     skips tiles where none of its keys is selected, and accumulates dv^T += dO^T P^T and
//     dk^T += Q^T dS^T into per-slice partials; dkv_reduce_kernel adds the slices in order.
//   Both kernels run every product on fp16 MFMA: Q, K, V and dO are converted to fp16 once per
//   call (to_f16_kernel; exact for bf16 values in fp16's normal range), and P and dS enter the
//   accumulations rounded to fp16 (2^-11 relative), one MFMA each instead of a bf16 hi + lo
//   pair.
#include "attn_tiles.h"

namespace dsa {

constexpr int kBwdSlice = 4096;  // query rows per dk/dv partial

// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ dout,
                                                        const uint16_t* __restrict__ out, int64_t n,
                                                        float* __restrict__ D) {
  const int64_t pair = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  float acc = 0.f;
  if (pair < n) {
    const i32x4 a = *reinterpret_cast<const i32x4*>(dout + pair * 128 + 8 * l);
    const i32x4 b = *reinterpret_cast<const i32x4*>(out + pair * 128 + 8 * l);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += bf16_to_f32(bf16_lane(a, e)) * bf16_to_f32(bf16_lane(b, e));
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o);
  if (pair < n && l == 0) D[pair] = acc;
}

// ------------------------------------------------------------------------------------------
// Selection bitmap: for 32-row block j of sequence b, W[woff_b + j L_b + s] has bit r set when
// row 32j + r selected key s (s <= 32j + 31).  woff_b = sum over earlier sequences of
// ceil(L/32) L.
// ------------------------------------------------------------------------------------------
constexpr int kBitmapChunk = 16384;

__device__ __forceinline__ int64_t bitmap_offset(const int32_t* __restrict__ cu, int b) {
  int64_t off = 0;
  for (int x = 0; x < b; ++x) {
    const int64_t L = cu[x + 1] - cu[x];
    off += ((L + 31) / 32) * L;
  }
  return off;
}

__global__ __launch_bounds__(256) void sel_bitmap_kernel(const int32_t* __restrict__ idx, int K,
                                                         const int32_t* __restrict__ cu,
                                                         const int2* __restrict__ sched,
                                                         const int* __restrict__ count, uint32_t* __restrict__ W) {
  __shared__ uint32_t words[kBitmapChunk];
  __shared__ int rbeg[32], rend[32];
  const int n = blockIdx.x;
  if (n >= *count) return;
  const int2 e = sched[n];
  const int b = e.x, j = e.y;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int i0 = 32 * j, nr = min(32, L - i0), plast = i0 + nr - 1;
  uint32_t* __restrict__ wrow = W + bitmap_offset(cu, b) + (int64_t)j * L;
  const int tid = threadIdx.x;
  if (tid < 32) rbeg[tid] = 0;
  for (int c0 = 0; c0 <= plast; c0 += kBitmapChunk) {
    const int c1 = c0 + kBitmapChunk;
    for (int i = tid; i < kBitmapChunk; i += 256) words[i] = 0u;
    if (tid < nr) {
      const int32_t* row = idx + (seq0 + i0 + tid) * K;
      int lo = rbeg[tid], hi = min(K, i0 + tid + 1);
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (row[mid] < c1) lo = mid + 1; else hi = mid;
      }
      rend[tid] = lo;
    }
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
      const int32_t* row = idx + (seq0 + i0 + r) * K;
      for (int x = rbeg[r] + tid; x < rend[r]; x += 256) atomicOr(&words[row[x] - c0], 1u << r);
    }
    __syncthreads();
    const int cend = min(plast + 1, c1) - c0;
    for (int i = tid; i < cend; i += 256) wrow[c0 + i] = words[i];
    if (tid < nr) rbeg[tid] = rend[tid];
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// X^T G^T accumulation for one 64-row tile: X^T (dims x rows) read transposed from an fp16 LDS
// tile, G (in the S^T register layout) rounded to fp16, one MFMA per step.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void accumulate_xt_gt_f16(const uint8_t* xl, const float (&gz)[2][16], int lane,
                                                     f32x16 (&o)[4]) {
  const int grp = lane >> 4, jj = lane & 15;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const i32x4 ph = pack_f16x8(&gz[rb][8 * kk2]);
      const int key_a = 32 * rb + 16 * kk2 + 8 * (grp >> 1) + (jj >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int dim0 = 32 * db + 16 * (grp & 1) + 4 * (jj & 3);
        const s16x4 a0 = lds_tr16(xl + kv_off(key_a, 2 * dim0));
        const s16x4 a1 = lds_tr16(xl + kv_off(key_a + 4, 2 * dim0));
        const i32x4 a = __builtin_bit_cast(i32x4, (s16x8_t){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        o[db] = mfma_f16_32x32x16(a, ph, o[db]);
      }
    }
}

// bf16 -> fp16 copy of n8 16-byte units (exact for values in fp16's normal range).
__global__ __launch_bounds__(256) void to_f16_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                     int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const i32x4 x = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(in) + i);
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = bf16_to_f32(bf16_lane(x, e));
  reinterpret_cast<i32x4*>(out)[i] = pack_f16x8(f);
}

// ------------------------------------------------------------------------------------------
// dedup_dq_kernel<G, SUB>: q, k, v, dout are the fp16 copies.  One workgroup per (16-row block,
// group of G query heads), G/2 waves,
// as the dedup attention kernel (same union, masks and mapping).  SUB groups share one KV head:
// 16 query heads per KV head run as two 8-head workgroups (one 8-wave workgroup would be
// limited to 256 registers per wave and spill).
// ------------------------------------------------------------------------------------------
constexpr int kDqRows = 16;

template <int G, int SUB>
__global__ __launch_bounds__(32 * G) void dedup_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dlt,
    const int32_t* __restrict__ cu, int Hq, int Hkv, float scale_log2, float scale, const int2* __restrict__ sched,
    const int* __restrict__ sched_count, int64_t ustride, const int32_t* __restrict__ ukeys,
    const uint16_t* __restrict__ umask, const int* __restrict__ ucount, float* __restrict__ dq) {
  constexpr int D = 128, BN = 64, NTH = 32 * G, UPT = 1024 / NTH, RW = 32 / G;
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "a wave's 32 query vectors must span whole rows");
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2][2][kKvTileB];  // [buffer][K=0/V=1], fp16
  __shared__ int upos[2][BN];
  const int n = blockIdx.x / (Hkv * SUB);
  const int gv = blockIdx.x % (Hkv * SUB);  // query-head group
  const int g = gv / SUB;                    // its KV head
  if (n >= *sched_count) return;
  const int2 e = sched[n];
  const int b = e.x, j = e.y;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int i0 = kDqRows * j;
  const int nr = min(kDqRows, L - i0);
  const int U = ucount[n];
  const int32_t* __restrict__ uk = ukeys + (int64_t)n * ustride;
  const uint16_t* __restrict__ um = umask + (int64_t)n * ustride;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int qc = lane & 31, hf = lane >> 5;
  const int qv = 32 * w + qc;
  const int my_r = qv / G;
  const int head = gv * G + qv % G;
  const int rbase = (32 * w) / G;
  const int64_t kvs = (int64_t)Hkv * D;
  const int64_t trow = seq0 + i0 + min(my_r, nr - 1);

  i32x4 qf[8], df[8];
  {
    const uint16_t* qp = q + (trow * Hq + head) * D + 8 * hf;
    const uint16_t* dp = dout + (trow * Hq + head) * D + 8 * hf;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      qf[s2] = *reinterpret_cast<const i32x4*>(qp + 16 * s2);
      df[s2] = *reinterpret_cast<const i32x4*>(dp + 16 * s2);
    }
  }
  const float lse2 = lse[trow * Hq + head] * 1.4426950408889634f;
  const float dlt = Dlt[trow * Hq + head];
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

  i32x4 pre[2 * UPT];
  auto gload = [&](const int* pos) {
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + NTH * x;
      const int64_t row = seq0 + pos[u >> 4];
      pre[x] = *reinterpret_cast<const i32x4*>(k + row * kvs + g * D + 8 * (u & 15));
      pre[UPT + x] = *reinterpret_cast<const i32x4*>(v + row * kvs + g * D + 8 * (u & 15));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + NTH * x;
      const int off = kv_off(u >> 4, 16 * (u & 15));
      *reinterpret_cast<i32x4*>(&kv_lds[buf][0][off]) = pre[x];
      *reinterpret_cast<i32x4*>(&kv_lds[buf][1][off]) = pre[UPT + x];
    }
  };

  if (U > 0) {
    if (tid < BN) {
      upos[0][tid] = uk[min(tid, U - 1)];
      upos[1][tid] = uk[min(BN + tid, U - 1)];
    }
    __syncthreads();
    gload(upos[0]);
    lstore(0);
  }
  __syncthreads();
  int buf = 0, t = 0;
  for (int u0 = 0; u0 < U; u0 += BN, ++t) {
    const bool more = u0 + BN < U;
    if (more) gload(upos[(t + 1) & 1]);
    const int pos2 = (tid < BN) ? uk[min(u0 + 2 * BN + tid, U - 1)] : 0;
    const int mk = (u0 + lane < U) ? int(um[u0 + lane]) : 0;
    uint64_t myword = 0;
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      const uint64_t bw = __ballot((mk >> (rbase + rr)) & 1);
      if (my_r == rbase + rr) myword = bw;
    }
    const uint64_t mw = myword >> (8 * hf);
    const uint32_t mlo = uint32_t(mw), mhi = uint32_t(mw >> 32);
    const uint8_t* kl = kv_lds[buf][0];
    const uint8_t* vl = kv_lds[buf][1];
    float gz[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = 0.f;
        pacc[i] = 0.f;
      }
      const int key = 32 * rb + kperm(qc);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        sacc = mfma_f16_32x32x16(*reinterpret_cast<const i32x4*>(kl + kv_off(key, 32 * s2 + 16 * hf)), qf[s2], sacc);
        pacc = mfma_f16_32x32x16(*reinterpret_cast<const i32x4*>(vl + kv_off(key, 32 * s2 + 16 * hf)), df[s2], pacc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t bit = 1u << (16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3));
        const bool on = ((rb ? mhi : mlo) & bit) != 0u;
        const float p = on ? __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -lse2)) : 0.f;
        gz[rb][i] = p * (pacc[i] - dlt);
      }
    }
    accumulate_xt_gt_f16(kl, gz, lane, o);
    if (more) lstore(buf ^ 1);
    if (tid < BN) upos[t & 1][tid] = pos2;
    __syncthreads();
    buf ^= 1;
  }
  if (my_r >= nr) return;
  float* op = dq + ((seq0 + i0 + my_r) * Hq + head) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<f32x4*>(op + 32 * db + 8 * a + 4 * hf) =
          (f32x4){o[db][4 * a] * scale, o[db][4 * a + 1] * scale, o[db][4 * a + 2] * scale, o[db][4 * a + 3] * scale};
}

// ------------------------------------------------------------------------------------------
// sparse_dkv_kernel<G>: grid (128-key blocks, KV heads, row slices), 4 waves x 32 keys; q, k,
// v, dout are the fp16 copies.
// ------------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void sparse_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dlt,
    const int32_t* __restrict__ cu, int Hq, int Hkv, float scale_log2, float scale, const int2* __restrict__ sched,
    const int* __restrict__ count, const uint32_t* __restrict__ W, int64_t T, float* __restrict__ dk_part,
    float* __restrict__ dv_part) {
  constexpr int D = 128, BN = 64, RT = BN / G;  // query vectors and rows per tile
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "tiles of whole rows inside a 32-row block");
  __shared__ __attribute__((aligned(16))) uint8_t t_lds[2][2][kKvTileB];  // [buffer][Q=0/dO=1], fp16
  __shared__ float stat[2][2][BN];                                          // [buffer][lse2, D][vector]
  const int n = blockIdx.x;
  if (n >= *count) return;
  const int2 e = sched[n];
  const int b = e.x, g = blockIdx.y, slice = blockIdx.z;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int s0 = 128 * e.y;
  const int t_lo = max(s0, slice * kBwdSlice), t_hi = min(L, (slice + 1) * kBwdSlice);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 31, hf = lane >> 5;
  const int my_s = s0 + 32 * w + qc;
  const bool valid = my_s < L;
  const int srow = min(my_s, L - 1);
  const int64_t kvs = (int64_t)Hkv * D;
  const uint32_t* __restrict__ wseq = W + bitmap_offset(cu, b);
  f32x16 dka[4], dva[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[db][i] = 0.f;
      dva[db][i] = 0.f;
    }
  if (t_lo < t_hi) {
    i32x4 kf[8], vf[8];
    {
      const uint16_t* kp = k + (seq0 + srow) * kvs + g * D + 8 * hf;
      const uint16_t* vp = v + (seq0 + srow) * kvs + g * D + 8 * hf;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        kf[s2] = *reinterpret_cast<const i32x4*>(kp + 16 * s2);
        vf[s2] = *reinterpret_cast<const i32x4*>(vp + 16 * s2);
      }
    }
    i32x4 pre[8];
    float spre[2];
    auto gload = [&](int t0) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int u = tid + 256 * x;  // vector u >> 4 = (row, head) (u >> 4) / G, (u >> 4) % G
        const int vv = u >> 4;
        const int64_t tr = seq0 + min(t0 + vv / G, t_hi - 1);
        const int64_t off = (tr * Hq + g * G + vv % G) * D + 8 * (u & 15);
        pre[x] = *reinterpret_cast<const i32x4*>(q + off);
        pre[4 + x] = *reinterpret_cast<const i32x4*>(dout + off);
      }
      if (tid < BN) {
        const int64_t tr = seq0 + min(t0 + tid / G, t_hi - 1);
        spre[0] = lse[tr * Hq + g * G + tid % G] * 1.4426950408889634f;
        spre[1] = Dlt[tr * Hq + g * G + tid % G];
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int u = tid + 256 * x;
        const int off = kv_off(u >> 4, 16 * (u & 15));
        *reinterpret_cast<i32x4*>(&t_lds[buf][0][off]) = pre[x];
        *reinterpret_cast<i32x4*>(&t_lds[buf][1][off]) = pre[4 + x];
      }
      if (tid < BN) {
        stat[buf][0][tid] = spre[0];
        stat[buf][1][tid] = spre[1];
      }
    };
    // selection bits of this lane's key for the 32-row block holding row t0
    auto bits_of = [&](int t0) -> uint32_t {
      const int rb = t0 >> 5;
      if (!valid || my_s > 32 * rb + 31) return 0u;
      const uint32_t word = wseq[(int64_t)rb * L + my_s];
      return (RT == 32) ? word : ((word >> (t0 & 31)) & ((1u << RT) - 1u));
    };
    gload(t_lo);
    lstore(0);
    uint32_t nbits = bits_of(t_lo);
    __syncthreads();
    int buf = 0;
    for (int t0 = t_lo; t0 < t_hi; t0 += RT) {
      const bool more = t0 + RT < t_hi;
      const uint32_t mybits = nbits;
      if (more) {
        gload(t0 + RT);
        nbits = bits_of(t0 + RT);
      }
      if (__any(mybits != 0u)) {
        const uint8_t* ql = t_lds[buf][0];
        const uint8_t* dl = t_lds[buf][1];
        float pz[2][16], sz[2][16];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x16 sacc, pacc;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            sacc[i] = 0.f;
            pacc[i] = 0.f;
          }
          const int vrow = 32 * rb + kperm(qc);
#pragma unroll
          for (int s2 = 0; s2 < 8; ++s2) {
            sacc = mfma_f16_32x32x16(*reinterpret_cast<const i32x4*>(ql + kv_off(vrow, 32 * s2 + 16 * hf)), kf[s2],
                                     sacc);
            pacc = mfma_f16_32x32x16(*reinterpret_cast<const i32x4*>(dl + kv_off(vrow, 32 * s2 + 16 * hf)), vf[s2],
                                     pacc);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int vl = 32 * rb + kperm(8 * (i >> 2) + 4 * hf + (i & 3));  // vector within the tile
            const bool on = (mybits >> (vl / G)) & 1u;
            const float p = on ? __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -stat[buf][0][vl])) : 0.f;
            pz[rb][i] = p;
            sz[rb][i] = p * (pacc[i] - stat[buf][1][vl]);
          }
        }
        accumulate_xt_gt_f16(dl, pz, lane, dva);
        accumulate_xt_gt_f16(ql, sz, lane, dka);
      }
      if (more) lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
  if (!valid) return;
  const int64_t orow = ((int64_t)slice * T + seq0 + my_s) * Hkv + g;
  float* kp = dk_part + orow * D;
  float* vp = dv_part + orow * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dim = 32 * db + 8 * a + 4 * hf;
      *reinterpret_cast<f32x4*>(kp + dim) = (f32x4){dka[db][4 * a] * scale, dka[db][4 * a + 1] * scale,
                                                    dka[db][4 * a + 2] * scale, dka[db][4 * a + 3] * scale};
      *reinterpret_cast<f32x4*>(vp + dim) =
          (f32x4){dva[db][4 * a], dva[db][4 * a + 1], dva[db][4 * a + 2], dva[db][4 * a + 3]};
    }
}

// dk/dv[row] = sum of the row's slice partials in slice order (slices whose rows all precede the
// key hold no contribution and are skipped).
__global__ __launch_bounds__(128) void dkv_reduce_kernel(const float* __restrict__ dk_part,
                                                         const float* __restrict__ dv_part,
                                                         const int32_t* __restrict__ cu, int nseq, int64_t T, int Hkv,
                                                         float* __restrict__ dk, float* __restrict__ dv) {
  const int64_t row = blockIdx.x;
  const int g = blockIdx.y;
  const int b = find_seq(cu, nseq, row);
  const int s = int(row - cu[b]);
  const int L = cu[b + 1] - cu[b];
  const int first = s / kBwdSlice, nsl = (L + kBwdSlice - 1) / kBwdSlice;
  float ak = 0.f, av = 0.f;
  for (int sl = first; sl < nsl; ++sl) {
    const int64_t o = (((int64_t)sl * T + row) * Hkv + g) * 128 + threadIdx.x;
    ak += dk_part[o];
    av += dv_part[o];
  }
  const int64_t o = (row * Hkv + g) * 128 + threadIdx.x;
  dk[o] = ak;
  dv[o] = av;
}

// ------------------------------------------------------------------------------------------
int bwd_slices(int max_len) { return (max_len + kBwdSlice - 1) / kBwdSlice; }

hipError_t launch_bwd_delta(const uint16_t* dout, const uint16_t* out, int64_t pairs, float* D, hipStream_t st) {
  if (pairs == 0) return hipSuccess;
  bwd_delta_kernel<<<(unsigned)((pairs + 15) / 16), 256, 0, st>>>(dout, out, pairs, D);
  return hipGetLastError();
}

hipError_t launch_sel_bitmap(const int32_t* idx, int K, const int32_t* cu, const int2* sched32, const int* count32,
                             int nb32, uint32_t* W, hipStream_t st) {
  if (nb32 == 0) return hipSuccess;
  sel_bitmap_kernel<<<nb32, 256, 0, st>>>(idx, K, cu, sched32, count32, W);
  return hipGetLastError();
}

hipError_t launch_dedup_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                           const float* lse, const float* Dlt, const int32_t* cu, int Hq, int Hkv, float scale,
                           const int2* sched16, const int* count16, int nb16, int64_t ustride, const int32_t* ukeys,
                           const uint16_t* umask, const int* ucount, float* dq, hipStream_t st) {
  if (nb16 == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  const unsigned grid = (unsigned)(nb16 * Hkv);
  switch (Hq / Hkv) {
#define DSA_DQ(GG, SUB)                                                                                             \
  dedup_dq_kernel<GG, SUB><<<grid * SUB, 32 * GG, 0, st>>>(q, k, v, dout, lse, Dlt, cu, Hq, Hkv, sl2, scale, sched16, \
                                                          count16, ustride, ukeys, umask, ucount, dq);
    case 2: DSA_DQ(2, 1) break;
    case 4: DSA_DQ(4, 1) break;
    case 8: DSA_DQ(8, 1) break;
    case 16: DSA_DQ(8, 2) break;
#undef DSA_DQ
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// fp16 copy of n elements (a multiple of 8) of bf16.
hipError_t launch_to_f16(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t st) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  to_f16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(in, out, n8);
  return hipGetLastError();
}

// q, k, v, dout: the fp16 copies.
hipError_t launch_sparse_dkv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                             const float* lse, const float* Dlt, const int32_t* cu, int nseq, int Hq, int Hkv,
                             float scale, const int2* sched128, const int* count128, int nb128, const uint32_t* W,
                             int max_len, int64_t T, float* dk_part, float* dv_part, float* dk, float* dv,
                             hipStream_t st) {
  if (T == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 grid(nb128, Hkv, bwd_slices(max_len));
  switch (Hq / Hkv) {
#define DSA_DKV(GG)                                                                                                \
  case GG:                                                                                                         \
    sparse_dkv_kernel<GG><<<grid, 256, 0, st>>>(q, k, v, dout, lse, Dlt, cu, Hq, Hkv, sl2, scale, sched128, count128, \
                                                W, T, dk_part, dv_part);                                           \
    break;
    DSA_DKV(2)
    DSA_DKV(4)
    DSA_DKV(8)
    DSA_DKV(16)
#undef DSA_DKV
    default:
      return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dkv_reduce_kernel<<<dim3((unsigned)T, Hkv), 128, 0, st>>>(dk_part, dv_part, cu, nseq, T, Hkv, dk, dv);
  return hipGetLastError();
}

}  // namespace dsa
