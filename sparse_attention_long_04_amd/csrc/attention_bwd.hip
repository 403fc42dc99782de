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
// Selection bitmap: for 32-row block j of sequence b, W[woff_b + j Lp_b + s] has bit r set
// when row 32j + r selected key s (s <= 32j + 31), Lp = L rounded up to a multiple of 4 (so
// that every block's 128 words start 16-byte aligned).  woff_b = sum over earlier sequences of
// ceil(L/32) Lp.
// ------------------------------------------------------------------------------------------
constexpr int kBitmapChunk = 16384;

__device__ __forceinline__ int64_t bitmap_offset(const int32_t* __restrict__ cu, int b) {
  int64_t off = 0;
  for (int x = 0; x < b; ++x) {
    const int64_t L = cu[x + 1] - cu[x];
    off += ((L + 31) / 32) * ((L + 3) & ~int64_t(3));
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
  uint32_t* __restrict__ wrow = W + bitmap_offset(cu, b) + (int64_t)j * ((L + 3) & ~3);
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
// X^T G^T accumulation for rows 32 rb .. 32 rb + 31 of a 64-row tile: X^T (dims x rows) read
// transposed from an fp16 LDS tile, G (in the S^T register layout) rounded to fp16, one MFMA
// per step.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void accumulate_xt_gt_f16(const uint8_t* xl, const float (&gz)[16], int rb, int lane,
                                                     f32x16 (&o)[4]) {
  const int grp = lane >> 4, jj = lane & 15;
#pragma unroll
  for (int kk2 = 0; kk2 < 2; ++kk2) {
    const i32x4 ph = pack_f16x8(&gz[8 * kk2]);
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
__global__ __launch_bounds__(32 * G, G == 8 ? 2 : 1) void dedup_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dlt,
    const int32_t* __restrict__ cu, int Hq, int Hkv, float scale_log2, float scale, const int2* __restrict__ sched,
    const int* __restrict__ sched_count, int64_t ustride, const int32_t* __restrict__ ukeys,
    const uint16_t* __restrict__ umask, const int* __restrict__ ucount, float* __restrict__ dq) {
  constexpr int D = 128, BN = 64, NTH = 32 * G, RW = 32 / G;
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "a wave's 32 query vectors must span whole rows");
  __shared__ __attribute__((aligned(1024))) uint8_t kv_lds[2][2][kKvTileB];  // [buffer][K=0/V=1], fp16
  __shared__ int upos[2][BN], umk[2][BN];  // union positions and row masks of upcoming tiles
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

  // K and V rows of the next tile, copied straight into LDS: copy x of this wave fills rows
  // 4 (CPW w + x) + lane/16 of the tile, LDS unit lane % 16 holding unit (lane % 16) ^ s(row)
  // (the kv_off swizzle); the positions come from upos.
  constexpr int CPW = 16 / (NTH / 64);  // 1 KB copies per wave and matrix
  lds_u8* const lb = (lds_u8*)&kv_lds[0][0][0];
  const uint32_t lds0 = (uint32_t)(uintptr_t)lb;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint16_t* const kg = k + seq0 * kvs + g * D;
  const uint16_t* const vg = v + seq0 * kvs + g * D;
  const uint32_t rowb = uint32_t(kvs) * 2;
  auto copies = [&](int slot, int buf) {
#pragma unroll
    for (int x = 0; x < CPW; ++x) {
      const int r = 4 * (CPW * wu + x) + (lane >> 4);
      const int sw = ((r & 3) << 2) | ((r >> 2) & 3);
      const uint32_t off = uint32_t(upos[slot][r]) * rowb + 16 * ((lane & 15) ^ sw);
      const uint32_t dst = lds0 + buf * 2 * kKvTileB + 1024 * (CPW * wu + x);
      dn_copy16(kg, off, dst);
      dn_copy16(vg, off, dst + kKvTileB);
    }
  };

  if (U > 0) {
    if (tid < BN) {
      upos[0][tid] = uk[min(tid, U - 1)];
      upos[1][tid] = uk[min(BN + tid, U - 1)];
      umk[0][tid] = (tid < U) ? int(um[tid]) : 0;
    }
    __syncthreads();
    copies(0, 0);
  }
  dn_sync();  // tile 0 has landed
  int t = 0;
  for (int u0 = 0; u0 < U; u0 += BN, ++t) {
    const int buf = t & 1;
    if (u0 + BN < U) copies(buf ^ 1, buf ^ 1);
    // positions of tile t+2 and masks of tile t+1, stored at the end of the iteration
    int pos2 = 0, mk1 = 0;
    if (tid < BN) {
      pos2 = uk[min(u0 + 2 * BN + tid, U - 1)];
      mk1 = (u0 + BN + tid < U) ? int(um[u0 + BN + tid]) : 0;
    }
    const int mk = umk[buf][lane];
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
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {  // keys 32 rb .. 32 rb + 31 of the tile: S, dP, dS, dq^T += K^T dS^T
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
      float gz[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t bit = 1u << (16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3));
        const bool on = ((rb ? mhi : mlo) & bit) != 0u;
        const float p = __builtin_amdgcn_exp2f(on ? fmaf(sacc[i], scale_log2, -lse2) : -__builtin_inff());
        gz[i] = p * (pacc[i] - dlt);
      }
      accumulate_xt_gt_f16(kl, gz, rb, lane, o);
    }
    if (tid < BN) {
      upos[buf][tid] = pos2;
      umk[buf ^ 1][tid] = mk1;
    }
    dn_sync();  // tile t+1 has landed; everyone is past tile t
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
// Column layout of the dk/dv pass: vector (row t, head h) of KV group g of sequence b is column
// bwd_col_base(cu[b], G, b) + G t + h of that group's transposed fp16 Q and dO copies
// ([g][dim][column]) and of its statistics ([g][-lse log2 e | -D][column]).  Each sequence
// starts on a 64-column boundary; its last 64-column tile is padded with zeros.
// ------------------------------------------------------------------------------------------
__device__ __host__ __forceinline__ int64_t bwd_col_base(int64_t cub, int G, int b) {
  return (cub * G + 63) / 64 * 64 + 64 * int64_t(b);
}
int64_t bwd_cols(int64_t T, int G, int nseq) { return bwd_col_base(T, G, nseq); }

// fp16 copies of q and dout in both layouts, and the statistics, for 64 columns of one KV group
// (block (c, g)); thread (vg, u) converts dims 8u .. 8u+7 of the block's vectors 8vg .. 8vg+7.
// The natural copies cover every (row, head) exactly once over the grid.
__global__ __launch_bounds__(128) void bwd_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ Dlt, const int32_t* __restrict__ cu, int nseq, int Hq, int G, int64_t ncols,
    uint16_t* __restrict__ qh, uint16_t* __restrict__ doh, uint16_t* __restrict__ qt,
    uint16_t* __restrict__ dot, float* __restrict__ stats) {
  const int64_t c0 = 64 * (int64_t)blockIdx.x;
  const int g = blockIdx.y;
  int lo = 0, hi = nseq - 1;  // the last sequence whose columns start at or before c0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bwd_col_base(cu[mid], G, mid) <= c0) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int64_t j0 = c0 - bwd_col_base(seq0, G, b);
  if (j0 >= ((int64_t)L * G + 63) / 64 * 64) return;  // between two sequences' columns
  const int tid = threadIdx.x, u = tid & 15, vg = tid >> 4;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const uint16_t* __restrict__ src = pass ? dout : q;
    uint16_t* __restrict__ nat = pass ? doh : qh;
    uint16_t* __restrict__ tr = pass ? dot : qt;
    float f[8][8];
#pragma unroll
    for (int vi = 0; vi < 8; ++vi) {
      const int64_t j = j0 + 8 * vg + vi;
      const int64_t t = j / G;
      if (t < L) {
        const int64_t off = ((seq0 + t) * Hq + g * G + int(j % G)) * 128 + 8 * u;
        const i32x4 x = *reinterpret_cast<const i32x4*>(src + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[vi][e] = bf16_to_f32(bf16_lane(x, e));
        *reinterpret_cast<i32x4*>(nat + off) = pack_f16x8(f[vi]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[vi][e] = 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float col[8];
#pragma unroll
      for (int vi = 0; vi < 8; ++vi) col[vi] = f[vi][e];
      *reinterpret_cast<i32x4*>(tr + (int64_t(g) * 128 + 8 * u + e) * ncols + c0 + 8 * vg) = pack_f16x8(col);
    }
  }
  if (tid < 64) {
    const int64_t j = j0 + tid, t = j / G;
    float a = 0.f, d = 0.f;
    if (t < L) {
      const int64_t r = (seq0 + t) * Hq + g * G + int(j % G);
      a = -lse[r] * 1.4426950408889634f;
      d = -Dlt[r];
    }
    stats[int64_t(g) * 2 * ncols + c0 + tid] = a;
    stats[(int64_t(g) * 2 + 1) * ncols + c0 + tid] = d;
  }
}

// ------------------------------------------------------------------------------------------
// sparse_dkv_kernel<G>: grid (128-key blocks, KV heads, row slices), 8 waves: waves 0-3 (the
// producers) and waves 4-7 (the consumers) share key group w % 4 (32 keys, the MFMA columns).
// The rows of the slice stream through LDS in half tiles of 32 (row, head) vectors, copied
// straight from global memory into two rings: the S ring (4 slots, filled by the producers:
// fp16 Q and dO rows, the A operands of S^T = K Q^T and dP^T = V dO^T, plus -lse log2 e and -D
// of each vector and the 128 keys' selection words) and the A ring (3 slots, filled by the
// consumers: the transposed fp16 Q^T and dO^T, the A operands of dk^T += Q^T dS^T and
// dv^T += dO^T P^T).  In iteration h a producer computes S and dP of half tile h+1 while it
// turns S and dP of half tile h into P = 2^(S scale log2 e - lse log2 e) (masked by the
// selection bits) and dS = P (dP - D), rounded to fp16 into an exchange buffer; its consumer
// accumulates the dk/dv products of half tile h-1 from the other exchange buffer.  One barrier
// per iteration; the copies run three (S) and two (A) half tiles ahead.
// ------------------------------------------------------------------------------------------
constexpr int kDkvS = 17408;                     // S slot: Q rows | dO rows (32 x 256 B each) | small
constexpr int kDkvSmall = 16384;                 // -lse log2 e [32] | -D [32] | words [128] | spare [64]
constexpr int kDkvA = 16384;                     // A slot: Q^T | dO^T (128 dims x 64 B each)
constexpr int kDkvAring = 4 * kDkvS;             // A ring offset
constexpr int kDkvX = kDkvAring + 3 * kDkvA;     // exchange buffers: [2][key group][P0 P1 dS0 dS1][64 lanes][16 B]
constexpr int kDkvLds = kDkvX + 2 * 4 * 4096;    // 151552 bytes
constexpr int kDkvCopiesS = 5;                   // copies per producer and iteration
constexpr int kDkvCopiesA = 4;                   // copies per consumer and iteration

template <int G>
__global__ __launch_bounds__(512) void sparse_dkv_kernel(
    const uint16_t* __restrict__ qh, const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vh,
    const uint16_t* __restrict__ doh, const uint16_t* __restrict__ qt, const uint16_t* __restrict__ dot,
    const float* __restrict__ stats, int64_t ncols, const int32_t* __restrict__ cu, int Hq, int Hkv,
    float scale_log2, float scale, const int2* __restrict__ sched, const int* __restrict__ count,
    const uint32_t* __restrict__ W, int64_t T, float* __restrict__ dk_part, float* __restrict__ dv_part) {
  constexpr int D = 128, RH = 32 / G;  // rows per half tile
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "half tiles of whole rows inside a 32-row block");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kDkvLds];
  const int n = blockIdx.x;
  if (n >= *count) return;
  const int2 e = sched[n];
  const int b = e.x, g = blockIdx.y, slice = blockIdx.z;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int s0 = 128 * e.y;
  const int t_lo = max(s0, slice * kBwdSlice), t_hi = min(L, (slice + 1) * kBwdSlice);
  const int tid = threadIdx.x, lane = tid & 63, qc = lane & 31, hf = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = wv & 3;                 // key group
  const bool producer = wv < 4;
  const int my_s = s0 + 32 * w + qc;
  const bool valid = my_s < L;
  lds_u8* const lb = (lds_u8*)lds;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lb;
  const int nh = (t_hi - t_lo + RH - 1) / RH;  // half tiles (0 if the slice holds none of the block's rows)
  auto tile_row = [&](int x) { return t_lo + RH * min(x, nh - 1); };
  const int64_t cb = bwd_col_base(seq0, G, b);

  if (producer) {
    if (nh <= 0) return;
    const int srow = min(my_s, L - 1);
    const int64_t kvs = (int64_t)Hkv * D;
    // K and V of the lane's key (B operands of S^T and dP^T): dims 16 s2 + 8 hf .. +7
    i32x4 kf[8], vf[8];
    {
      const uint16_t* kp = kh + (seq0 + srow) * kvs + g * D + 8 * hf;
      const uint16_t* vp = vh + (seq0 + srow) * kvs + g * D + 8 * hf;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        kf[s2] = *reinterpret_cast<const i32x4*>(kp + 16 * s2);
        vf[s2] = *reinterpret_cast<const i32x4*>(vp + 16 * s2);
      }
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) asm volatile("" : "+v"(kf[s2]), "+v"(vf[s2]));  // landed before any copy
    }
    const uint16_t* const qnb = qh + (seq0 * Hq + g * G) * D;  // row r, head hh: + (r Hq + hh) D
    const uint16_t* const dnb = doh + (seq0 * Hq + g * G) * D;
    const float* const stb = stats + int64_t(g) * 2 * ncols + cb;
    const int Lp = (L + 3) & ~3;
    const uint32_t* const wb = W + bitmap_offset(cu, b) + s0;
    // S part x (clamped to the last half tile): rows 4(2w + i) + lane/16 of the Q and dO stages,
    // 16-byte unit (lane % 16) holding unit (lane % 16) ^ (row % 16); small region: lanes 0..15
    // fill bytes 256 w .. (wave 0: -lse log2 e and -D, waves 1 and 2: the words of keys 0..63 and
    // 64..127, wave 3: a spare copy of the statistics).  Five copies per producer.
    const uint32_t sm_off = (w == 1 || w == 2) ? uint32_t(256 * (w - 1) + 16 * (lane & 15))
                                               : ((lane & 8) ? uint32_t(ncols) * 4 : 0u) + 16 * (lane & 7);
    auto copies_s = [&](int x) {
      const int t0 = tile_row(x);
      const uint32_t slot = lds0 + (x & 3) * kDkvS;
      const void* src = (w == 1 || w == 2) ? (const void*)(wb + int64_t(t0 >> 5) * Lp) : (const void*)(stb + int64_t(G) * t0);
      dn_copy16_lo16(src, sm_off, slot + kDkvSmall + 256 * w);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int vi = 4 * (2 * w + i) + (lane >> 4);
        const int r = min(t0 + vi / G, t_hi - 1);
        const uint32_t off = uint32_t(r * Hq + vi % G) * 256 + 16 * ((lane & 15) ^ (vi & 15));
        dn_copy16(qnb, off, slot + 1024 * (2 * w + i));
        dn_copy16(dnb, off, slot + 8192 + 1024 * (2 * w + i));
      }
    };
    // S operand reads: row kperm(qc), unit 2 s2 + hf -> byte qn_off ^ 32 s2 (slot offsets are
    // multiples of 64, so the unit XOR commutes with them)
    const int vrow = kperm(qc);
    const int qn_off = 256 * vrow + 16 * (hf ^ (vrow & 15));
    // statistics of the lane's accumulator rows (vectors 16(j/2) + 8 hf + 4(j%2) .. +3, j < 4)
    float lc[16], dc[16];
    auto load_stats = [&](int x) {
      const lds_u8* sm = lb + (x & 3) * kDkvS + kDkvSmall;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v0 = 16 * (j >> 1) + 8 * hf + 4 * (j & 1);
        const f32x4 a = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(sm + 4 * v0);
        const f32x4 c = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(sm + 128 + 4 * v0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          lc[4 * j + m] = a[m];
          dc[4 * j + m] = c[m];
        }
      }
    };
    // selection bits of the lane's key for the rows of half tile x, shifted so that bit r / G of
    // the result belongs to accumulator register i (r = 16(i/8) + 4((i/4)%2) + i%4)
    auto load_bits = [&](int x) -> uint32_t {
      const int t0 = t_lo + RH * x;
      const uint32_t word = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(
          lb + (x & 3) * kDkvS + kDkvSmall + 256 + 4 * (32 * w + qc));
      const uint32_t keep = (valid && my_s <= 32 * (t0 >> 5) + 31) ? 0xFFFFFFFFu : 0u;
      const uint32_t bits = (word >> (t0 & 31)) & ((1u << RH) - 1u) & keep;
      return (G == 16) ? bits : (bits >> ((8 * hf) / G));
    };
    // S and dP of half tile x into (s, p), operand reads two MFMAs ahead
    auto chains = [&](int x, f32x16& s, f32x16& p) {
      const int sq = (x & 3) * kDkvS + qn_off;
      i32x4 op[16];
      auto rd = [&](auto jj) {
        constexpr int j = decltype(jj)::value;
        op[j] = dn_ld128(lb + (sq ^ (32 * (j >> 1))) + ((j & 1) ? 8192 : 0));
      };
      rd(dn_ic<0>{});
      rd(dn_ic<1>{});
      auto step = [&](auto jj) {
        constexpr int j = decltype(jj)::value;
        if constexpr (j + 2 < 16) rd(dn_ic<j + 2>{});
        if constexpr (j & 1) p = mfma_f16_32x32x16(op[j], vf[j >> 1], (j >> 1) ? p : (f32x16){});
        else s = mfma_f16_32x32x16(op[j], kf[j >> 1], (j >> 1) ? s : (f32x16){});
      };
      step(dn_ic<0>{});  step(dn_ic<1>{});  step(dn_ic<2>{});  step(dn_ic<3>{});
      step(dn_ic<4>{});  step(dn_ic<5>{});  step(dn_ic<6>{});  step(dn_ic<7>{});
      step(dn_ic<8>{});  step(dn_ic<9>{});  step(dn_ic<10>{}); step(dn_ic<11>{});
      step(dn_ic<12>{}); step(dn_ic<13>{}); step(dn_ic<14>{}); step(dn_ic<15>{});
    };
    // one producer iteration: S, dP of half tile h+1 (16 MFMAs) with P and dS of half tile h
    // (element i in slot i) computed between them; P and dS go to exchange buffer h % 2
    auto body = [&](int h, const f32x16& sc, const f32x16& pc, f32x16& sn, f32x16& pn) {
      copies_s(h + 3);
      load_stats(h);
      const uint32_t bh = load_bits(h);
      const int sq = ((h + 1) & 3) * kDkvS + qn_off;
      i32x4 op[16];
      i32x4 ppk[2], dpk[2];
      float pv[2], dv2[2];
      auto rd = [&](auto jj) {
        constexpr int j = decltype(jj)::value;
        op[j] = dn_ld128(lb + (sq ^ (32 * (j >> 1))) + ((j & 1) ? 8192 : 0));
      };
      auto ev = [&](auto ii) {
        constexpr int i = decltype(ii)::value;
        constexpr int r = 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
        const bool on = (bh >> (r / G)) & 1u;
        const float p = __builtin_amdgcn_exp2f(on ? fmaf(sc[i], scale_log2, lc[i]) : -__builtin_inff());
        pv[i & 1] = p;
        dv2[i & 1] = p * (pc[i] + dc[i]);
        if constexpr (i & 1) {
          const f16x2 hp = {(_Float16)pv[0], (_Float16)pv[1]};
          const f16x2 hd = {(_Float16)dv2[0], (_Float16)dv2[1]};
          int xp = __builtin_bit_cast(int, hp), xd = __builtin_bit_cast(int, hd);
          asm volatile("" : "+v"(xp), "+v"(xd));  // computed in this slot
          ppk[i >> 3][(i & 7) >> 1] = xp;
          dpk[i >> 3][(i & 7) >> 1] = xd;
        }
      };
      rd(dn_ic<0>{});
      rd(dn_ic<1>{});
      auto slot = [&](auto jj) {
        constexpr int j = decltype(jj)::value;
        if constexpr (j + 2 < 16) rd(dn_ic<j + 2>{});
        if constexpr (j & 1) pn = mfma_f16_32x32x16(op[j], vf[j >> 1], (j >> 1) ? pn : (f32x16){});
        else sn = mfma_f16_32x32x16(op[j], kf[j >> 1], (j >> 1) ? sn : (f32x16){});
        ev(dn_ic<j>{});
        __builtin_amdgcn_sched_barrier(0);
      };
      slot(dn_ic<0>{});  slot(dn_ic<1>{});  slot(dn_ic<2>{});  slot(dn_ic<3>{});
      slot(dn_ic<4>{});  slot(dn_ic<5>{});  slot(dn_ic<6>{});  slot(dn_ic<7>{});
      slot(dn_ic<8>{});  slot(dn_ic<9>{});  slot(dn_ic<10>{}); slot(dn_ic<11>{});
      slot(dn_ic<12>{}); slot(dn_ic<13>{}); slot(dn_ic<14>{}); slot(dn_ic<15>{});
      __attribute__((address_space(3))) i32x4* xb =
          reinterpret_cast<__attribute__((address_space(3))) i32x4*>(lb + kDkvX + (h & 1) * 16384 + 4096 * w) + lane;
      xb[0] = ppk[0];
      xb[64] = ppk[1];
      xb[128] = dpk[0];
      xb[192] = dpk[1];
      lds_sync_vm<kDkvCopiesS>();  // S part h+2 has landed; the exchange buffer is written
    };
    // prologue: S parts 0..1 land (part 2 stays in flight); S(0), dP(0)
    copies_s(0);
    copies_s(1);
    copies_s(2);
    lds_sync_vm<kDkvCopiesS>();
    f32x16 sa, pa, sb, pb2;
    chains(0, sa, pa);
    int h = 0;
    for (; h + 1 < nh; h += 2) {
      body(h, sa, pa, sb, pb2);
      body(h + 1, sb, pb2, sa, pa);
    }
    if (h < nh) {
      body(h, sa, pa, sb, pb2);
      ++h;
    }
    // iteration nh: the consumers take the last half tile
    copies_s(nh + 3);
    lds_sync_vm<kDkvCopiesS>();
    dn_sync();  // no copy is left in flight when the workgroup ends
    return;
  }

  // ---- consumers: dk^T += Q^T dS^T, dv^T += dO^T P^T of half tile h-1 in iteration h
  f32x16 dka[4], dva[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dka[db] = (f32x16){};
    dva[db] = (f32x16){};
  }
  if (nh > 0) {
    const uint16_t* const qtb = qt + int64_t(g) * D * ncols + cb;  // dim d, vector j: + d ncols + j
    const uint16_t* const dtb = dot + int64_t(g) * D * ncols + cb;
    // A part x (clamped): dim rows 16(2w + i) + lane/4, unit (lane % 4) holding unit
    // (lane % 4) ^ ((dim / 4) % 4).  Four copies per consumer.
    uint32_t at_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = 16 * (2 * w + i) + (lane >> 2);
      at_off[i] = uint32_t(d) * uint32_t(ncols) * 2 + 16 * ((lane & 3) ^ ((d >> 2) & 3));
    }
    auto copies_a = [&](int x) {
      const int64_t c0 = int64_t(G) * tile_row(x);
      const uint32_t slot = lds0 + kDkvAring + (x % 3) * kDkvA;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        dn_copy16(qtb + c0, at_off[i], slot + 1024 * (2 * w + i));
        dn_copy16(dtb + c0, at_off[i], slot + 8192 + 1024 * (2 * w + i));
      }
    };
    // operand reads: dim row 32 db + qc, unit 2 kk + hf -> byte 2048 db + (qa_off ^ 32 kk)
    const int qa_off = 64 * qc + 16 * (hf ^ ((qc >> 2) & 3));
    auto body = [&](int x) {  // the products of half tile x
      const int aq = kDkvAring + (x % 3) * kDkvA + qa_off;
      const __attribute__((address_space(3))) i32x4* xb =
          reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(lb + kDkvX + (x & 1) * 16384 + 4096 * w) +
          lane;
      const i32x4 ppk[2] = {xb[0], xb[64]};
      const i32x4 dpk[2] = {xb[128], xb[192]};
      i32x4 op[16];
      auto rd = [&](auto jj) {  // MFMA j: kk = j / 8, db = (j % 8) / 2, dv (j even, dO^T) or dk (Q^T)
        constexpr int j = decltype(jj)::value;
        op[j] = dn_ld128(lb + (aq ^ (32 * (j >> 3))) + ((j & 1) ? 0 : 8192) + 2048 * ((j & 7) >> 1));
      };
      rd(dn_ic<0>{});
      rd(dn_ic<1>{});
      rd(dn_ic<2>{});
      auto step = [&](auto jj) {
        constexpr int j = decltype(jj)::value;
        constexpr int kk = j >> 3, db = (j & 7) >> 1;
        if constexpr (j + 3 < 16) rd(dn_ic<j + 3>{});
        if constexpr (j & 1) dka[db] = mfma_f16_32x32x16(op[j], dpk[kk], dka[db]);
        else dva[db] = mfma_f16_32x32x16(op[j], ppk[kk], dva[db]);
      };
      step(dn_ic<0>{});  step(dn_ic<1>{});  step(dn_ic<2>{});  step(dn_ic<3>{});
      step(dn_ic<4>{});  step(dn_ic<5>{});  step(dn_ic<6>{});  step(dn_ic<7>{});
      step(dn_ic<8>{});  step(dn_ic<9>{});  step(dn_ic<10>{}); step(dn_ic<11>{});
      step(dn_ic<12>{}); step(dn_ic<13>{}); step(dn_ic<14>{}); step(dn_ic<15>{});
    };
    // prologue: A part 0 in flight (it lands by the end of iteration 0)
    copies_a(0);
    lds_sync_vm<kDkvCopiesA>();
    for (int h = 0; h <= nh; ++h) {
      copies_a(h + 1);
      if (h > 0) body(h - 1);
      lds_sync_vm<kDkvCopiesA>();  // A part h has landed; this wave is past exchange buffer h-1
    }
    dn_sync();
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
                           const uint16_t* umask, const int* ucount, float* dq, int max_len, hipStream_t st) {
  if (nb16 == 0) return hipSuccess;
  // the K/V copy offsets are 32-bit byte offsets from the sequence's first row
  if (int64_t(max_len) * Hkv * 256 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
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

// fp16 Q and dO in both layouts and the statistics of the dk/dv pass (after launch_bwd_delta).
hipError_t launch_bwd_prep(const uint16_t* q, const uint16_t* dout, const float* lse, const float* Dlt,
                           const int32_t* cu, int nseq, int64_t T, int Hq, int Hkv, uint16_t* qh, uint16_t* doh,
                           uint16_t* qt, uint16_t* dot, float* stats, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t ncols = bwd_cols(T, G, nseq);
  bwd_prep_kernel<<<dim3((unsigned)(ncols / 64), Hkv), 128, 0, st>>>(q, dout, lse, Dlt, cu, nseq, Hq, G, ncols, qh, doh,
                                                                   qt, dot, stats);
  return hipGetLastError();
}

// qh, kh, vh, doh: the natural fp16 copies; qt, dot, stats: launch_bwd_prep's outputs.
hipError_t launch_sparse_dkv(const uint16_t* qh, const uint16_t* kh, const uint16_t* vh, const uint16_t* doh,
                             const uint16_t* qt, const uint16_t* dot, const float* stats, const int32_t* cu, int nseq,
                             int Hq, int Hkv, float scale, const int2* sched128, const int* count128, int nb128,
                             const uint32_t* W, int max_len, int64_t T, float* dk_part, float* dv_part, float* dk,
                             float* dv, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int G = Hq / Hkv;
  const int64_t ncols = bwd_cols(T, G, nseq);
  // the kernel's copy offsets are 32-bit: rows of one sequence, and 128 transposed dim rows
  if (int64_t(max_len) * Hq * 256 >= (int64_t(1) << 32) || 256 * ncols >= (int64_t(1) << 32))
    return hipErrorInvalidValue;
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 grid(nb128, Hkv, bwd_slices(max_len));
  switch (G) {
#define DSA_DKV(GG)                                                                                              \
  case GG:                                                                                                       \
    sparse_dkv_kernel<GG><<<grid, 512, 0, st>>>(qh, kh, vh, doh, qt, dot, stats, ncols, cu, Hq, Hkv, sl2, scale,  \
                                                sched128, count128, W, T, dk_part, dv_part);                     \
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
