// Dense warm-up objective of the Lightning Indexer (Keye-VL-2.0 summary page, gsyq.cn, section
// 一: while the full attention stays unchanged, the indexer is trained so that its judgement of
// which positions matter follows the full attention's distribution; the gap is a KL divergence
// that is minimised).
//
// Per query token t (keys s <= t of its sequence):
//     p_t = mean over the Hq query heads of softmax_s(scale q[t,h] . k[s, g(h)])   (target)
//     r_t = softmax_s(I[t, :]),  I = the Lightning Indexer scores
//     KL_t = sum_s p log(p / r),   g[t, s] = r - p  (gradient of KL_t with respect to I[t, s])
// and, with c[t,h,s] = q_I[t,h] . k_I[s], the gradients of sum_t KL_t with respect to the indexer
// inputs:
//     dw[t,h]  = sum_s g[t,s] max(0, c)
//     dq_I[t,h] = w[t,h] sum_s g[t,s] [c > 0] k_I[s]
//     dk_I[s]  = sum_{t >= s} sum_h g[t,s] w[t,h] [c > 0] q_I[t,h]
//
// Kernels (all rows of one sequence; packed sequences via cu_seqlens):
//   kl_lse_kernel     per (128 query rows, query head): log-sum-exp of the scaled scores (log2
//                     units) -- the dense kernel's S^T = K Q^T tile loop with an online max/sum.
//   kl_target_kernel  per 128-key chunk x 128 query rows: p += 2^(S_h - lse_h) summed over all
//                     Hq heads in registers (one KV head's K rows staged in LDS at a time),
//                     written once into a score-shaped triangle (16-row blocks, as the indexer's
//                     scores).
//   kl_row_kernel     per row: softmax statistics of the indexer row, KL_t, then g = r - p in
//                     place of p.
//   kl_dq_kernel      per block of 256/H_I rows: the dense kernel's loop over 64-key tiles with
//                     the H_I x rows query vectors as MFMA columns; S^T = k_I q_I^T (fp8 MFMA on
//                     the e4m3 codes, exact), G = g [S > 0] in registers, dq^T += k_I^T G^T (bf16
//                     MFMA, G split hi + lo), dw accumulated from the same registers; the head
//                     weight scales the finished row.
//   kl_dk_kernel      roles swapped: per 256 keys x a slice of the query rows, 64-vector tiles of
//                     (row, head) pairs, G = g w [S > 0]; dk^T += q_I^T G^T into per-slice
//                     partials.
//   kl_dk_reduce_kernel  sums the partials in slice order (deterministic; no float atomics).
#include "attn_tiles.h"

namespace dsa {

// Row i of a sequence's score-shaped triangle starting at tri + off (16-row blocks, row stride
// 16 (block + 1) floats).
__device__ __forceinline__ const float* tri_row(const float* tri, int64_t off, int i) {
  const int j = i >> 4;
  return tri + off + score_block_offset(j) + (i & 15) * 16 * (int64_t)(j + 1);
}

// e4m3 (OCP, bias 7) codes are exact in fp32 and bf16.  The conversions below use the hardware's
// fp8 -> fp32 pair conversion (two codes of a 16-bit half of a dword), then keep the upper halves
// of the two floats (bf16, an exact truncation).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <bool UPPER>
__device__ __forceinline__ f32x2_t e4m3x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(int(word), UPPER);
}
__device__ __forceinline__ int bf16_pair(f32x2_t f) {
  return int(__builtin_amdgcn_perm(__float_as_uint(f.y), __float_as_uint(f.x), 0x07060302u));
}

// 16 e4m3 codes (a uint4) -> 16 bf16, 2 x 4 dwords (code order).
__device__ __forceinline__ void e4m3x16_to_bf16(uint4 v, i32x4 (&bf)[2]) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    bf[wi >> 1][2 * (wi & 1)] = bf16_pair(e4m3x2_to_f32<false>(w4[wi]));
    bf[wi >> 1][2 * (wi & 1) + 1] = bf16_pair(e4m3x2_to_f32<true>(w4[wi]));
  }
}

// ------------------------------------------------------------------------------------------
// kl_lse_kernel: grid (128-row blocks, Hq), 4 waves x 32 query rows of one head.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void kl_lse_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                     const int32_t* __restrict__ cu, int Hq, int Hkv, float scale_log2,
                                                     const int2* __restrict__ sched, const int* __restrict__ count,
                                                     float* __restrict__ lse) {
  constexpr int D = 128, BN = 64;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][kKvTileB];
  const int n = blockIdx.x;
  if (n >= *count) return;
  const int2 e = sched[n];
  const int b = e.x, h = blockIdx.y, g = h / (Hq / Hkv);
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int q0 = 128 * e.y, kend = min(L, q0 + 128);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 31, hf = lane >> 5;
  const int my_q = q0 + 32 * w + qc;
  const int wave_qmax = q0 + 32 * w + 31;
  const int wave_qmin = q0 + 32 * __builtin_amdgcn_readfirstlane(w);  // tiles ending before it need no mask
  const int64_t kvs = (int64_t)Hkv * D;
  i32x4 qf[8];
  {
    const uint16_t* qp = q + ((seq0 + min(my_q, kend - 1)) * Hq + h) * D + 8 * hf;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) qf[s2] = *reinterpret_cast<const i32x4*>(qp + 16 * s2);
  }
  i32x4 pre[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int u = tid + 256 * x;
      const int kk = min(kt + (u >> 4), kend - 1);
      pre[x] = *reinterpret_cast<const i32x4*>(k + (seq0 + kk) * kvs + g * D + 8 * (u & 15));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int u = tid + 256 * x;
      *reinterpret_cast<i32x4*>(&k_lds[buf][kv_off(u >> 4, 16 * (u & 15))]) = pre[x];
    }
  };
  float m_run = -__builtin_inff(), l_run = 0.f;
  gload(0);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int kt = 0; kt < kend; kt += BN) {
    const bool more = kt + BN < kend;
    if (more) gload(kt + BN);
    if (kt <= wave_qmax) {
      // raw scores; the running max is kept in raw units (scale > 0), so each score costs one
      // fma before its exponential, and keys are masked only on tiles that reach the diagonal
      f32x16 z[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) z[rb][i] = 0.f;
        const int key = 32 * rb + kperm(qc);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          z[rb] = mfma_bf16_32x32x16(*reinterpret_cast<const i32x4*>(&k_lds[buf][kv_off(key, 32 * s2 + 16 * hf)]),
                                     qf[s2], z[rb]);
      }
      if (kt + BN - 1 > wave_qmin) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kt + 32 * rb + kperm(8 * (i >> 2) + 4 * hf + (i & 3)) > my_q) z[rb][i] = -__builtin_inff();
      }
      float mt = fmaxf(z[0][0], z[1][0]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, z[rb][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float msc = m_use * scale_log2;
      float ps = 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) ps += __builtin_amdgcn_exp2f(fmaf(z[rb][i], scale_log2, -msc));
      l_run = l_run * __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2) + ps;
      m_run = m_new;
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_q < kend && hf == 0) lse[(seq0 + my_q) * Hq + h] = m_run * scale_log2 + __log2f(l_tot);
}

// ------------------------------------------------------------------------------------------
// kl_target_kernel: grid (128-key chunks, 128-row blocks; chunks vary fastest, so the
// workgroups resident together read the same rows' queries from L2), 4 waves x 32 query rows,
// two workgroups per CU.  The chunk's p sums stay in registers (4 tiles x 16 per lane) for all
// Hq heads: per KV head, its 128 K rows are copied into LDS (two buffers, the next KV head's copy
// in flight during the current one), and every query head of the group takes its Q fragment from
// global memory once per chunk (the next head's prefetched) for the 4 tiles.  Any Hq / HKV works.
// ------------------------------------------------------------------------------------------
constexpr int kKlTargetChunk = 128;

template <int HKV>
__global__ __launch_bounds__(256, 2) void kl_target_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                        const int32_t* __restrict__ cu, int Hq, float scale_log2,
                                                        const int2* __restrict__ sched, const int* __restrict__ count,
                                                        const float* __restrict__ lse,
                                                        const int64_t* __restrict__ seqoff, float* __restrict__ P) {
  constexpr int D = 128, BN = 32, KC = kKlTargetChunk, NT = KC / BN, TB = KC * kKvRowB;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][TB];
  const int n = blockIdx.y;
  if (n >= *count) return;
  const int2 e = sched[n];
  const int b = e.x;
  const int G = Hq / HKV;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int q0 = 128 * e.y, kend = min(L, q0 + 128);
  // this workgroup's key chunk (the rows' outputs are independent across key ranges)
  const int kbeg = KC * blockIdx.x;
  if (kbeg >= kend) return;
  const int kstop = min(kend, kbeg + KC);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 31, hf = lane >> 5;
  const int my_q = q0 + 32 * w + qc;
  const int qrow = min(my_q, kend - 1);
  // tiles of the chunk that reach this wave's rows (none for a wave entirely before the chunk)
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const int wlast = min(q0 + 32 * ws + 31, kstop - 1);
  const int nt = wlast < kbeg ? 0 : (wlast - kbeg) / BN + 1;
  // K copy: wave w fills rows KC w / 4 + 4 x + lane / 16 of a buffer, one 16-byte unit per lane, for
  // the tiles any wave reads (rows past the sequence's end repeat its last key; their scores
  // are never written).  Byte offsets from the sequence's first row fit 32 bits (the launcher
  // checks the K size).
  const int crows = BN * ((kstop - kbeg + BN - 1) / BN);
  const uint32_t rowb = uint32_t(HKV * D * 2);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&k_lds[0][0];
  constexpr int CPW = KC / 16;  // 4-row copies per wave
  auto copy_k = [&](int g, int kb) {
    const uint16_t* kg = k + seq0 * (HKV * D) + g * D;
#pragma unroll
    for (int x = 0; x < CPW; ++x) {
      const int r = 4 * CPW * w + 4 * x + (lane >> 4);
      if (4 * CPW * ws + 4 * x < crows) {
        const uint32_t kr = uint32_t(min(kbeg + r, kend - 1));
        const int swz = ((r & 3) << 2) | ((r >> 2) & 3);
        dn_copy16(kg, kr * rowb + 16 * ((lane & 15) ^ swz), lds0 + kb * TB + 1024 * (CPW * ws + x));
      }
    }
  };
  // queries of head h for this lane's row: 8 x 16 bytes (dims 16 s2 + 8 hf ..), and its lse
  const uint16_t* const qrow_p = q + (seq0 + qrow) * Hq * D + 8 * hf;
  const float* const lse_row = lse + (seq0 + qrow) * Hq;
  auto qload = [&](i32x4 (&dst)[8], float& ls, int h) {
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) dst[s2] = *reinterpret_cast<const i32x4*>(qrow_p + h * D + 16 * s2);
    ls = lse_row[h];
  };
  float pacc[NT][16];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) pacc[t][i] = 0.f;
  const int key = kperm(qc);
  auto head = [&](const i32x4 (&qf)[8], float ls, int kb) {
    const uint8_t* kl = k_lds[kb];
    auto scores = [&](int t) {
      f32x16 sacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2)
        sacc = mfma_bf16_32x32x16(*reinterpret_cast<const i32x4*>(kl + kv_off(BN * t + key, 32 * s2 + 16 * hf)),
                                  qf[s2], sacc);
      return sacc;
    };
    auto accumulate = [&](int t, const f32x16& sacc) {
#pragma unroll
      for (int i = 0; i < 16; ++i) pacc[t][i] += __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -ls));
    };
    if (nt == NT) {
      // every tile: tile t + 1's products are issued before tile t's exponentials, so the
      // matrix core and the vector unit overlap
      f32x16 cur = scores(0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x16 nxt;
        if (t + 1 < NT) nxt = scores(t + 1);
        accumulate(t, cur);
        if (t + 1 < NT) cur = nxt;
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t < nt) accumulate(t, scores(t));
    }
  };
  // heads in order (each one's successor loaded while it is computed); at the first head of KV
  // group g, its K rows have landed and every wave is done with the other buffer, which then
  // receives group g + 1's rows
  auto step = [&](int h, const i32x4 (&cur)[8], float lc, i32x4 (&nxt)[8], float& ln) {
    const int g = h / G;
    if (h % G == 0) {
      dn_sync();
      if (g + 1 < HKV) copy_k(g + 1, (g + 1) & 1);
    }
    qload(nxt, ln, min(h + 1, Hq - 1));
    head(cur, lc, g & 1);
  };
  i32x4 qa[8], qb[8];
  float la, lb;
  copy_k(0, 0);
  qload(qa, la, 0);
  for (int h = 0; h < Hq; h += 2) {
    step(h, qa, la, qb, lb);
    if (h + 1 < Hq) step(h + 1, qb, lb, qa, la);
  }
  // C row (reg i, half hf) <-> key kbeg + 32 t + kperm(8(i/4) + 4hf + i%4): runs of 4 keys
  if (my_q < kend) {
    const float inv_hq = 1.f / float(Hq);
    float* prow = const_cast<float*>(tri_row(P, seqoff[b], qrow));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int k0 = kbeg + BN * t + kperm(8 * a + 4 * hf);
          if (k0 + 3 <= my_q) {
            *reinterpret_cast<f32x4*>(prow + k0) =
                (f32x4){pacc[t][4 * a] * inv_hq, pacc[t][4 * a + 1] * inv_hq, pacc[t][4 * a + 2] * inv_hq,
                        pacc[t][4 * a + 3] * inv_hq};
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (k0 + c <= my_q) prow[k0 + c] = pacc[t][4 * a + c] * inv_hq;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// kl_row_kernel: one workgroup per row.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kl_row_kernel(const float* __restrict__ I, float* __restrict__ P,
                                                     const int64_t* __restrict__ seqoff, const int32_t* __restrict__ cu,
                                                     int nseq, const float2* __restrict__ rowrange,
                                                     float* __restrict__ kl) {
  __shared__ float red[4][4];
  const int64_t t = blockIdx.x;
  const int b = find_seq(cu, nseq, t);
  const int i = int(t - cu[b]);
  const int nk = i + 1;
  const float* irow = tri_row(I, seqoff[b], i);
  float* prow = const_cast<float*>(tri_row(P, seqoff[b], i));
  const float mI = rowrange[t].y;
  float l = 0.f, sp = 0.f, splp = 0.f, spi = 0.f;
  for (int s = threadIdx.x; s < nk; s += 256) {
    const float x = irow[s], p = prow[s];
    l += __expf(x - mI);
    sp += p;
    spi += p * x;
    if (p > 0.f) splp += p * __logf(p);
  }
  float v[4] = {l, sp, splp, spi};
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    for (int o = 32; o > 0; o >>= 1) v[c] += __shfl_xor(v[c], o);
    if (lane == 0) red[c][w] = v[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = red[c][0] + red[c][1] + red[c][2] + red[c][3];
  const float lse_i = mI + __logf(v[0]);
  if (threadIdx.x == 0) kl[t] = v[2] - v[3] + lse_i * v[1];
  const float inv_l = 1.f / v[0];
  for (int s = threadIdx.x; s < nk; s += 256) prow[s] = __expf(irow[s] - mI) * inv_l - prow[s];
}

// ------------------------------------------------------------------------------------------
// Shared by the two gradient kernels: a 64-row tile of e4m3 rows (128 codes each) staged in LDS
// twice -- the raw codes (128 bytes per row: the fp8 MFMA operand of the score recompute) and
// the same rows as bf16 (256 bytes per row in the K/V layout: read transposed as the first
// operand of the G contraction).  Unit u (16 bytes) of a raw row r sits at u ^ ((r / 2) % 8), so
// the 16 rows that a quarter wave reads at one unit fall on 16 distinct bank groups.
// ------------------------------------------------------------------------------------------
constexpr int kF8RowB = 128, kF8TileB = 64 * kF8RowB;
__device__ __forceinline__ int f8_off(int row, int unit) { return row * kF8RowB + 16 * (unit ^ ((row >> 1) & 7)); }

// 512 threads: thread -> row tid / 8, 16 codes (unit tid % 8).
__device__ __forceinline__ void fp8_tile_store(uint8_t* f8, uint8_t* bf, uint4 v, int tid) {
  const int r = tid >> 3, c = tid & 7;
  *reinterpret_cast<uint4*>(f8 + f8_off(r, c)) = v;
  i32x4 b[2];
  e4m3x16_to_bf16(v, b);
#pragma unroll
  for (int x = 0; x < 2; ++x) *reinterpret_cast<i32x4*>(bf + kv_off(r, 32 * c + 16 * x)) = b[x];
}

__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 32 e4m3 codes at p (16-byte aligned) as one fp8 MFMA operand.
__device__ __forceinline__ i32x8 load_f8x32(const uint8_t* p) {
  const i32x4 a = *reinterpret_cast<const i32x4*>(p), b = *reinterpret_cast<const i32x4*>(p + 16);
  return (i32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// S = (tile row `row`) . (lane column) over the 128 dims in two fp8 MFMAs: for step m, lane
// (c, hf) supplies dims 64 m + 32 hf .. + 31 of both operands (the same dims on both sides, so
// the sum does not depend on how the instruction orders them).
__device__ __forceinline__ f32x16 s_tile_f8(const uint8_t* f8, int row, int hf, const i32x8 (&col)[2]) {
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const i32x4 a0 = *reinterpret_cast<const i32x4*>(f8 + f8_off(row, 4 * m + 2 * hf));
    const i32x4 a1 = *reinterpret_cast<const i32x4*>(f8 + f8_off(row, 4 * m + 2 * hf + 1));
    acc = mfma_fp8_32x32x64((i32x8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}, col[m], acc);
  }
  return acc;
}

// 8 floats -> bf16 hi (each float's upper 16 bits) and lo (the exact remainder x - hi, again
// truncated to bf16), as packed pairs.  hi + lo keeps 16 or more significant bits of x, at any
// magnitude (bf16 has fp32's exponent range).
__device__ __forceinline__ void split_bf16x8(const float* x, i32x4& ph, i32x4& pl) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t u0 = __float_as_uint(x[2 * p]), u1 = __float_as_uint(x[2 * p + 1]);
    ph[p] = int(__builtin_amdgcn_perm(u1, u0, 0x07060302u));
    const float l0 = x[2 * p] - __uint_as_float(u0 & 0xFFFF0000u);
    const float l1 = x[2 * p + 1] - __uint_as_float(u1 & 0xFFFF0000u);
    pl[p] = int(__builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u));
  }
}

// O^T += X^T G^T for one 64-key tile: X^T (dims x keys) read transposed from the bf16 tile, G (in
// the S^T register layout) split into bf16 hi + lo.
__device__ __forceinline__ void accumulate_xt_gt(const uint8_t* xl, const float (&gz)[2][16], int lane,
                                                 f32x16 (&o)[4]) {
  const int grp = lane >> 4, jj = lane & 15;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      i32x4 ph, pl;
      split_bf16x8(&gz[rb][8 * kk2], ph, pl);
      const int key_a = 32 * rb + 16 * kk2 + 8 * (grp >> 1) + (jj >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int dim0 = 32 * db + 16 * (grp & 1) + 4 * (jj & 3);
        const s16x4 a0 = lds_tr16(xl + kv_off(key_a, 2 * dim0));
        const s16x4 a1 = lds_tr16(xl + kv_off(key_a + 4, 2 * dim0));
        const i32x4 a = __builtin_bit_cast(i32x4, (s16x8_t){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        o[db] = mfma_bf16_32x32x16(a, ph, o[db]);
        o[db] = mfma_bf16_32x32x16(a, pl, o[db]);
      }
    }
}

// ------------------------------------------------------------------------------------------
// kl_dq_kernel<HI>: grid (blocks of 256/HI rows), 8 waves; lane column = query vector
// v = 32 wave + c -> (row v / HI, head v % HI).  The head weight is applied once at the end
// (dq = w sum_s g [c > 0] k), so G here is g [c > 0].
// ------------------------------------------------------------------------------------------
template <int HI>
__global__ __launch_bounds__(512) void kl_dq_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx,
                                                    const float* __restrict__ wgt, const float* __restrict__ Gt,
                                                    const int64_t* __restrict__ seqoff, const int32_t* __restrict__ cu,
                                                    const int2* __restrict__ sched, const int* __restrict__ count,
                                                    float* __restrict__ dq, float* __restrict__ dw) {
  constexpr int D = 128, BN = 64, R = 256 / HI;
  static_assert(R % 4 == 0, "G rows are copied four at a time");
  __shared__ __attribute__((aligned(16))) uint8_t f8_lds[2][kF8TileB];
  __shared__ __attribute__((aligned(16))) uint8_t bf_lds[2][kKvTileB];
  __shared__ __attribute__((aligned(16))) float g_lds[2][R][BN];  // G of the block's rows for a key tile
  const int n = blockIdx.x;
  if (n >= *count) return;
  const int2 e = sched[n];
  const int b = e.x;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int r0 = R * e.y, kend = min(L, r0 + R);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 31, hf = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int v = 32 * w + qc;
  const int my_t = r0 + v / HI, head = v % HI;
  const bool valid = my_t < kend;
  const int trow = min(my_t, kend - 1);
  const int wave_tmax = min(kend - 1, r0 + (32 * wu + 31) / HI);
  // a tile needs no key mask for this wave when all its vectors are rows of the sequence and its
  // last key precedes the wave's first row
  const int wave_tmin = r0 + (32 * wu) / HI;
  const bool wave_full = r0 + (32 * wu + 31) / HI < kend;
  i32x8 qf[2];
  {
    const uint8_t* qp = q_idx + ((seq0 + trow) * HI + head) * D + 32 * hf;
#pragma unroll
    for (int m = 0; m < 2; ++m) qf[m] = load_f8x32(qp + 64 * m);
  }
  const float wq = wgt[(seq0 + trow) * HI + head];
  // G[t][kt .. kt+63] of the block's rows for key tile kt, copied into g_lds[gb] one tile ahead:
  // wave w < R/4 fills rows 4w .. 4w+3, 16 lanes per row (rows past the block end repeat its
  // last row and chunks past a row's stored width re-read its last chunk: both masked later)
  const int64_t soff = seqoff[b];
  const uint32_t glds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&g_lds[0][0][0];
  auto gcopy = [&](int kt, int gb) {
    if (wu < R / 4) {
      const int t = min(r0 + 4 * wu + (lane >> 4), kend - 1);
      const int width = 16 * ((t >> 4) + 1);  // stored floats of row t
      const int c = min(kt + 4 * (lane & 15), width - 4);
      const float* base = tri_row(Gt, soff, min(r0 + 4 * wu, kend - 1));
      const uint32_t off = uint32_t((tri_row(Gt, soff, t) - base) + c) * 4;
      dn_copy16(base, off, glds0 + (gb * R + 4 * wu) * BN * 4);
    }
  };
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float dwacc = 0.f;
  uint4 pre;
  auto gload = [&](int kt) {
    pre = *reinterpret_cast<const uint4*>(k_idx + (seq0 + min(kt + (tid >> 3), kend - 1)) * D + 16 * (tid & 7));
  };
  gload(0);
  gcopy(0, 0);
  fp8_tile_store(f8_lds[0], bf_lds[0], pre, tid);
  dn_sync();
  int buf = 0;
  for (int kt = 0; kt < kend; kt += BN) {
    const bool more = kt + BN < kend;
    if (more) {
      gload(kt + BN);
      gcopy(kt + BN, buf ^ 1);
    }
    if (kt <= wave_tmax) {
      const bool full = wave_full && kt + BN - 1 <= wave_tmin;
      float gz[2][16];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const f32x16 s = s_tile_f8(f8_lds[buf], 32 * rb + kperm(qc), hf, qf);
        // registers 4a .. 4a+3 <-> keys kt + kl0 .. kt + kl0 + 3 (consecutive)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int kl0 = 32 * rb + kperm(8 * a + 4 * hf);
          f32x4 g4 = *reinterpret_cast<const f32x4*>(&g_lds[buf][trow - r0][kl0]);
          if (!full) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (!valid || kt + kl0 + c > my_t) g4[c] = 0.f;
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float x = s[4 * a + c] > 0.f ? g4[c] : 0.f;
            gz[rb][4 * a + c] = x;
            dwacc = fmaf(x, s[4 * a + c], dwacc);  // g max(0, c)
          }
        }
      }
      accumulate_xt_gt(bf_lds[buf], gz, lane, o);
    }
    if (more) fp8_tile_store(f8_lds[buf ^ 1], bf_lds[buf ^ 1], pre, tid);
    dn_sync();  // the next tile's G has landed
    buf ^= 1;
  }
  dwacc += __shfl_xor(dwacc, 32);
  if (!valid) return;
  if (hf == 0) dw[(seq0 + my_t) * HI + head] = dwacc;
  float* op = dq + ((seq0 + my_t) * HI + head) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<f32x4*>(op + 32 * db + 8 * a + 4 * hf) =
          (f32x4){o[db][4 * a] * wq, o[db][4 * a + 1] * wq, o[db][4 * a + 2] * wq, o[db][4 * a + 3] * wq};
}

// ------------------------------------------------------------------------------------------
// kl_dk_kernel<HI>: grid (256-key blocks, query-row slices of kDkSlice rows), 8 waves; lane
// column = key s = s0 + 32 wave + c; tiles of 64 consecutive (row, head) vectors of the slice.
// G = g w [c > 0].  Writes partial dk [slice][T][128].
// ------------------------------------------------------------------------------------------
constexpr int kDkSlice = 1024;

template <int HI>
__global__ __launch_bounds__(512) void kl_dk_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx,
                                                    const float* __restrict__ wgt, const float* __restrict__ Gt,
                                                    const int64_t* __restrict__ seqoff, const int32_t* __restrict__ cu,
                                                    const int2* __restrict__ sched, const int* __restrict__ count,
                                                    int64_t T, float* __restrict__ dk_part) {
  constexpr int D = 128, BN = 64, RPT = BN / HI;  // rows per tile
  static_assert(HI >= 16 && HI <= 64, "a run of 4 vectors never crosses a row");
  __shared__ __attribute__((aligned(16))) uint8_t f8_lds[2][kF8TileB];
  __shared__ __attribute__((aligned(16))) uint8_t bf_lds[2][kKvTileB];
  __shared__ __attribute__((aligned(16))) float w_lds[2][BN];
  __shared__ __attribute__((aligned(16))) float g_lds[2][RPT][256];  // G of a tile's rows for the block's keys
  const int n = blockIdx.x;
  if (n >= *count) return;
  const int2 e = sched[n];
  const int b = e.x, slice = blockIdx.y;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int s0 = 256 * e.y, send = min(L, s0 + 256);
  const int t_lo = max(s0, slice * kDkSlice), t_hi = min(L, (slice + 1) * kDkSlice);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 31, hf = lane >> 5;
  const int my_s = s0 + 32 * w + qc;
  const bool valid = my_s < send;
  const int srow = min(my_s, send - 1);
  float* op = dk_part + ((int64_t)slice * T + seq0 + srow) * D;
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  if (t_lo < t_hi) {
    i32x8 kf[2];
    {
      const uint8_t* kp = k_idx + (seq0 + srow) * D + 32 * hf;
#pragma unroll
      for (int m = 0; m < 2; ++m) kf[m] = load_f8x32(kp + 64 * m);
    }
    const int64_t v_begin = (int64_t)t_lo * HI, v_end = (int64_t)t_hi * HI;  // vectors of this slice
    // G[t][s0 .. s0+255] of the tile's rows, copied into g_lds[gb] one tile ahead: wave w < RPT
    // fills row w, 4 keys per lane (rows past the slice repeat its last row and chunks past a
    // row's stored width re-read its last chunk: both masked later)
    const int64_t soff = seqoff[b];
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t glds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&g_lds[0][0][0];
    auto gcopy = [&](int64_t v0, int gb) {
      if (wu < RPT) {
        const int tr = min(int(v0 / HI) + wu, t_hi - 1);
        const int width = 16 * ((tr >> 4) + 1);  // stored floats of row tr
        const int c = min(s0 + 4 * lane, width - 4);
        dn_copy16(tri_row(Gt, soff, tr), uint32_t(c) * 4, glds0 + (gb * RPT + wu) * 1024);
      }
    };
    uint4 pre;
    float wpre = 0.f;
    auto gload = [&](int64_t v0) {
      const int64_t vv = min(v0 + (tid >> 3), v_end - 1);
      pre = *reinterpret_cast<const uint4*>(q_idx + (seq0 * HI + vv) * D + 16 * (tid & 7));
      if (tid < BN) wpre = wgt[seq0 * HI + min(v0 + tid, v_end - 1)];
    };
    auto lstore = [&](int buf) {
      fp8_tile_store(f8_lds[buf], bf_lds[buf], pre, tid);
      if (tid < BN) w_lds[buf][tid] = wpre;
    };
    gload(v_begin);
    gcopy(v_begin, 0);
    lstore(0);
    dn_sync();
    int buf = 0;
    for (int64_t v0 = v_begin; v0 < v_end; v0 += BN) {
      const bool more = v0 + BN < v_end;
      if (more) {
        gload(v0 + BN);
        gcopy(v0 + BN, buf ^ 1);
      }
      const int tt0 = int(v0 / HI);  // first row of the tile
      if (tt0 + RPT - 1 >= s0 + 32 * w) {  // some row of the tile sees some key of this wave
        // g[t, s] for the tile's rows (s <= t)
        float gr[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          const int tr = tt0 + r;
          gr[r] = (valid && tr < t_hi && my_s <= tr) ? g_lds[buf][r][32 * w + qc] : 0.f;
        }
        float gz[2][16];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const f32x16 s = s_tile_f8(f8_lds[buf], 32 * rb + kperm(qc), hf, kf);
          // registers 4a .. 4a+3 <-> vectors vl0 .. vl0 + 3 of the tile, all of row r
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int vl0 = 32 * rb + kperm(8 * a + 4 * hf);
            const int r = (32 * rb + 16 * (a >> 1) + 4 * (a & 1)) / HI;  // = vl0 / HI (8 hf < HI)
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(&w_lds[buf][vl0]);
#pragma unroll
            for (int c = 0; c < 4; ++c) gz[rb][4 * a + c] = s[4 * a + c] > 0.f ? gr[r] * w4[c] : 0.f;
          }
        }
        accumulate_xt_gt(bf_lds[buf], gz, lane, o);
      }
      if (more) lstore(buf ^ 1);
      dn_sync();  // the next tile's G has landed
      buf ^= 1;
    }
  }
  if (!valid) return;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<f32x4*>(op + 32 * db + 8 * a + 4 * hf) =
          (f32x4){o[db][4 * a], o[db][4 * a + 1], o[db][4 * a + 2], o[db][4 * a + 3]};
}

// dk[row] = sum over the row's slices (fixed order).  Slices that do not reach a row (all of
// their query rows precede it) were never written for it and are skipped.
__global__ __launch_bounds__(128) void kl_dk_reduce_kernel(const float* __restrict__ dk_part, const int32_t* __restrict__ cu,
                                                           int nseq, int64_t T, float* __restrict__ dk) {
  const int64_t row = blockIdx.x;
  const int b = find_seq(cu, nseq, row);
  const int s = int(row - cu[b]);
  const int L = cu[b + 1] - cu[b];
  const int first = s / kDkSlice, nsl = (L + kDkSlice - 1) / kDkSlice;
  float acc = 0.f;
  for (int sl = first; sl < nsl; ++sl) acc += dk_part[((int64_t)sl * T + row) * 128 + threadIdx.x];
  dk[row * 128 + threadIdx.x] = acc;
}

// ------------------------------------------------------------------------------------------
hipError_t launch_kl_lse(const uint16_t* q, const uint16_t* k, const int32_t* cu, int Hq, int Hkv, float scale,
                         const int2* sched128, const int* count128, int nb128, float* lse, hipStream_t st) {
  if (nb128 == 0) return hipSuccess;
  kl_lse_kernel<<<dim3(nb128, Hq), 256, 0, st>>>(q, k, cu, Hq, Hkv, scale * 1.4426950408889634f, sched128, count128,
                                                 lse);
  return hipGetLastError();
}

hipError_t launch_kl_target(const uint16_t* q, const uint16_t* k, const int32_t* cu, int Hq, int Hkv, float scale,
                            const int2* sched128, const int* count128, int nb128, int max_len, const float* lse,
                            const int64_t* seqoff, float* P, hipStream_t st) {
  if (nb128 == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  if ((int64_t)max_len * Hkv * 256 > 0xFFFFFFFFll) return hipErrorInvalidValue;  // 32-bit K copy offsets
  const dim3 grid((max_len + kKlTargetChunk - 1) / kKlTargetChunk, nb128);
  switch (Hkv) {
    case 1: kl_target_kernel<1><<<grid, 256, 0, st>>>(q, k, cu, Hq, sl2, sched128, count128, lse, seqoff, P); break;
    case 2: kl_target_kernel<2><<<grid, 256, 0, st>>>(q, k, cu, Hq, sl2, sched128, count128, lse, seqoff, P); break;
    case 4: kl_target_kernel<4><<<grid, 256, 0, st>>>(q, k, cu, Hq, sl2, sched128, count128, lse, seqoff, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kl_rows(const float* I, float* P, const int64_t* seqoff, const int32_t* cu, int nseq, int64_t T,
                          const float2* rowrange, float* kl, hipStream_t st) {
  if (T == 0) return hipSuccess;
  kl_row_kernel<<<(unsigned)T, 256, 0, st>>>(I, P, seqoff, cu, nseq, rowrange, kl);
  return hipGetLastError();
}

hipError_t launch_kl_dq(int H, const uint8_t* q_idx, const uint8_t* k_idx, const float* w, const float* G,
                        const int64_t* seqoff, const int32_t* cu, const int2* schedR, const int* countR, int nbR,
                        float* dq, float* dw, hipStream_t st) {
  if (nbR == 0) return hipSuccess;
  switch (H) {
    case 16: kl_dq_kernel<16><<<nbR, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, schedR, countR, dq, dw); break;
    case 32: kl_dq_kernel<32><<<nbR, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, schedR, countR, dq, dw); break;
    case 64: kl_dq_kernel<64><<<nbR, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, schedR, countR, dq, dw); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int kl_dk_slices(int max_len) { return (max_len + kDkSlice - 1) / kDkSlice; }

hipError_t launch_kl_dk(int H, const uint8_t* q_idx, const uint8_t* k_idx, const float* w, const float* G,
                        const int64_t* seqoff, const int32_t* cu, int nseq, const int2* sched256,
                        const int* count256, int nb256, int max_len, int64_t T, float* dk_part,
                        float* dk, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid(nb256, kl_dk_slices(max_len));
  switch (H) {
    case 16: kl_dk_kernel<16><<<grid, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, sched256, count256, T, dk_part); break;
    case 32: kl_dk_kernel<32><<<grid, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, sched256, count256, T, dk_part); break;
    case 64: kl_dk_kernel<64><<<grid, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, sched256, count256, T, dk_part); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  kl_dk_reduce_kernel<<<(unsigned)T, 128, 0, st>>>(dk_part, cu, nseq, T, dk);
  return hipGetLastError();
}

}  // namespace dsa
