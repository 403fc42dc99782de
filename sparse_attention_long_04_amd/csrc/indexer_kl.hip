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
//   kl_target_kernel  per 128 query rows: for each 32-key tile, p += 2^(S_h - lse_h) summed over
//                     all Hq heads (every KV head's K tile staged in LDS), written once into a
//                     score-shaped triangle (16-row blocks, as the indexer's scores).
//   kl_row_kernel     per row: softmax statistics of the indexer row, KL_t, then g = r - p in
//                     place of p.
//   kl_dq_kernel      per block of 256/H_I rows: the dense kernel's loop over 64-key tiles with
//                     the H_I x rows query vectors as MFMA columns; S^T = k_I q_I^T (bf16 MFMA,
//                     exact for e4m3 inputs), G = g w [S > 0] in registers, dq^T += k_I^T G^T
//                     (fp16 MFMA, G split hi + lo), dw accumulated from the same registers.
//   kl_dk_kernel      roles swapped: per 256 keys x a slice of the query rows, 64-vector tiles of
//                     (row, head) pairs; dk^T += q_I^T G^T into per-slice partials.
//   kl_dk_reduce_kernel  sums the partials in slice order (deterministic; no float atomics).
#include "attn_tiles.h"

namespace dsa {

// Row i of a sequence's score-shaped triangle starting at tri + off (16-row blocks, row stride
// 16 (block + 1) floats).
__device__ __forceinline__ const float* tri_row(const float* tri, int64_t off, int i) {
  const int j = i >> 4;
  return tri + off + score_block_offset(j) + (i & 15) * 16 * (int64_t)(j + 1);
}

// 8 e4m3 codes (a uint2) -> 8 bf16 (exact), packed as 4 dwords.
__device__ __forceinline__ i32x4 e4m3x8_to_bf16(uint2 v) {
  i32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t word = p < 2 ? v.x : v.y;
    const uint32_t b0 = (word >> (16 * (p & 1))) & 0xFFu, b1 = (word >> (16 * (p & 1) + 8)) & 0xFFu;
    r[p] = int((__float_as_uint(e4m3_decode(b0)) >> 16) | (__float_as_uint(e4m3_decode(b1)) & 0xFFFF0000u));
  }
  return r;
}

// 16 e4m3 codes (a uint4) -> 16 bf16 and 16 fp16 (both exact), 2 x 4 dwords each.
__device__ __forceinline__ void e4m3x16_convert(uint4 v, i32x4 (&bf)[2], i32x4 (&hf)[2]) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = e4m3_decode((w4[2 * half + (e >> 2)] >> (8 * (e & 3))) & 0xFFu);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      bf[half][p] = int((__float_as_uint(f[2 * p]) >> 16) | (__float_as_uint(f[2 * p + 1]) & 0xFFFF0000u));
    hf[half] = pack_f16x8(f);
  }
}

// ------------------------------------------------------------------------------------------
// kl_lse_kernel: grid (128-row blocks, Hq), 4 waves x 32 query rows of one head.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kl_lse_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
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
      float z[2][16];
      float mt = -__builtin_inff();
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
        const int key = 32 * rb + kperm(qc);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          sacc = mfma_bf16_32x32x16(*reinterpret_cast<const i32x4*>(&k_lds[buf][kv_off(key, 32 * s2 + 16 * hf)]),
                                    qf[s2], sacc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = kt + 32 * rb + kperm(8 * (i >> 2) + 4 * hf + (i & 3));
          z[rb][i] = (kk <= my_q) ? sacc[i] * scale_log2 : -__builtin_inff();
          mt = fmaxf(mt, z[rb][i]);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
      float ps = 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) ps += __builtin_amdgcn_exp2f(z[rb][i] - m_use);
      l_run = l_run * __builtin_amdgcn_exp2f(m_run - m_use) + ps;
      m_run = m_new;
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_q < kend && hf == 0) lse[(seq0 + my_q) * Hq + h] = m_run + __log2f(l_tot);
}

// ------------------------------------------------------------------------------------------
// kl_target_kernel: grid (128-row blocks, key chunks of kKlTargetChunk), 4 waves x 32 query
// rows, all heads; 32-key tiles of the HKV KV heads double-buffered in LDS.
// ------------------------------------------------------------------------------------------
constexpr int kKlTargetChunk = 2048;

template <int HKV>
__global__ __launch_bounds__(256) void kl_target_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                        const int32_t* __restrict__ cu, int Hq, float scale_log2,
                                                        const int2* __restrict__ sched, const int* __restrict__ count,
                                                        const float* __restrict__ lse,
                                                        const int64_t* __restrict__ seqoff, float* __restrict__ P) {
  constexpr int D = 128, BN = 32, TB = BN * kKvRowB, UPT = 2 * HKV;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][HKV][TB];
  const int n = blockIdx.x;
  if (n >= *count) return;
  const int2 e = sched[n];
  const int b = e.x;
  const int G = Hq / HKV;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int q0 = 128 * e.y, kend = min(L, q0 + 128);
  // this workgroup's key chunk (the rows' outputs are independent across key ranges)
  const int kbeg = kKlTargetChunk * blockIdx.y;
  if (kbeg >= kend) return;
  const int kstop = min(kend, kbeg + kKlTargetChunk);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 31, hf = lane >> 5;
  const int my_q = q0 + 32 * w + qc;
  const int qrow = min(my_q, kend - 1);
  const int wave_qmax = q0 + 32 * w + 31;
  const int64_t kvs = (int64_t)HKV * D;
  const float inv_hq = 1.f / float(Hq);
  i32x4 pre[UPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + 256 * x;  // head u / 512, key (u % 512) >> 4, column u & 15
      const int gg = u >> 9, kk = min(kt + ((u & 511) >> 4), kend - 1);
      pre[x] = *reinterpret_cast<const i32x4*>(k + (seq0 + kk) * kvs + gg * D + 8 * (u & 15));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + 256 * x;
      *reinterpret_cast<i32x4*>(&k_lds[buf][u >> 9][kv_off((u & 511) >> 4, 16 * (u & 15))]) = pre[x];
    }
  };
  const float* lse_row = lse + (seq0 + qrow) * Hq;
  float* prow = const_cast<float*>(tri_row(P, seqoff[b], qrow));
  gload(kbeg);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int kt = kbeg; kt < kstop; kt += BN) {
    const bool more = kt + BN < kstop;
    if (more) gload(kt + BN);
    if (kt <= wave_qmax) {
      float pacc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pacc[i] = 0.f;
      const int key = kperm(qc);
      i32x4 qa[8], qb[8];
      auto qload = [&](i32x4 (&dst)[8], int h) {
        const uint16_t* qp = q + ((seq0 + qrow) * Hq + h) * D + 8 * hf;
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) dst[s2] = *reinterpret_cast<const i32x4*>(qp + 16 * s2);
      };
      auto head = [&](const i32x4 (&qf)[8], int h) {
        const uint8_t* kl = k_lds[buf][h / G];
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          sacc = mfma_bf16_32x32x16(*reinterpret_cast<const i32x4*>(kl + kv_off(key, 32 * s2 + 16 * hf)), qf[s2],
                                    sacc);
        const float ls = lse_row[h];
#pragma unroll
        for (int i = 0; i < 16; ++i) pacc[i] += __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -ls));
      };
      // heads in pairs, the next pair's queries loaded while the current one is computed
      qload(qa, 0);
      for (int h = 0; h < Hq; h += 2) {
        qload(qb, h + 1);
        head(qa, h);
        if (h + 2 < Hq) qload(qa, h + 2);
        head(qb, h + 1);
      }
      // C row (reg i, half hf) <-> key kt + kperm(8(i/4) + 4hf + i%4): runs of 4 consecutive keys
      if (my_q < kend) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int k0 = kt + kperm(8 * a + 4 * hf);
          if (k0 + 3 <= my_q) {
            *reinterpret_cast<f32x4*>(prow + k0) = (f32x4){pacc[4 * a] * inv_hq, pacc[4 * a + 1] * inv_hq,
                                                           pacc[4 * a + 2] * inv_hq, pacc[4 * a + 3] * inv_hq};
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (k0 + c <= my_q) prow[k0 + c] = pacc[4 * a + c] * inv_hq;
          }
        }
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
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
// as bf16 (copy 0, MFMA A operand rows) and fp16 (copy 1, transposed second operand).
// 512 threads: thread -> row tid / 8, 16 codes at column 16 (tid % 8).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void fp8_tile_store(uint8_t* lds0, uint8_t* lds1, uint4 v, int tid) {
  i32x4 bf[2], hfv[2];
  e4m3x16_convert(v, bf, hfv);
  const int r = tid >> 3, c = tid & 7;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    *reinterpret_cast<i32x4*>(lds0 + kv_off(r, 32 * c + 16 * x)) = bf[x];
    *reinterpret_cast<i32x4*>(lds1 + kv_off(r, 32 * c + 16 * x)) = hfv[x];
  }
}

// Power-of-two pre-scale for the fp16 hi + lo split of G = g w [c > 0] (|g| <= 1): 2^(14 - e)
// with 2^e >= max |w|, so |G| scale <= 2^14 stays below fp16's maximum and small values stay
// normal.  gsc[0] = scale, gsc[1] = 1 / scale (both exact).  Two stages: kGscaleBlocks partial
// maxima, then one workgroup.
constexpr int kGscaleBlocks = 256;

__global__ __launch_bounds__(256) void kl_wmax_kernel(const float* __restrict__ w, int64_t n, float* __restrict__ part) {
  __shared__ float red[4];
  float m = 0.f;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += 256 * kGscaleBlocks) m = fmaxf(m, fabsf(w[i]));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(256) void kl_gscale_kernel(const float* __restrict__ part, float* __restrict__ gsc) {
  __shared__ float red[4];
  float m = part[threadIdx.x];
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (m > 0.f && m < __builtin_inff()) frexpf(m, &e);  // m = f 2^e, f in [1/2, 1): 2^e >= m
    e = max(-100, min(100, e));
    gsc[0] = ldexpf(1.f, 14 - e);
    gsc[1] = ldexpf(1.f, e - 14);
  }
}

// O^T += X^T G^T for one 64-key tile: X^T (dims x keys) read transposed from the fp16 tile, G (in
// the S^T register layout, already multiplied by the pre-scale) split into fp16 hi + lo.
__device__ __forceinline__ void accumulate_xt_gt(const uint8_t* xl, const float (&gz)[2][16], int lane,
                                                 f32x16 (&o)[4]) {
  const int grp = lane >> 4, jj = lane & 15;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      float hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = gz[rb][8 * kk2 + e];
        hi[e] = float(_Float16(x));
        lo[e] = x - hi[e];
      }
      const i32x4 ph = pack_f16x8(hi), pl = pack_f16x8(lo);
      const int key_a = 32 * rb + 16 * kk2 + 8 * (grp >> 1) + (jj >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int dim0 = 32 * db + 16 * (grp & 1) + 4 * (jj & 3);
        const s16x4 a0 = lds_tr16(xl + kv_off(key_a, 2 * dim0));
        const s16x4 a1 = lds_tr16(xl + kv_off(key_a + 4, 2 * dim0));
        const i32x4 a = __builtin_bit_cast(i32x4, (s16x8_t){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        o[db] = mfma_f16_32x32x16(a, ph, o[db]);
        o[db] = mfma_f16_32x32x16(a, pl, o[db]);
      }
    }
}

// ------------------------------------------------------------------------------------------
// kl_dq_kernel<HI>: grid (blocks of 256/HI rows), 8 waves; lane column = query vector
// v = 32 wave + c -> (row v / HI, head v % HI).
// ------------------------------------------------------------------------------------------
template <int HI>
__global__ __launch_bounds__(512) void kl_dq_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx,
                                                    const float* __restrict__ wgt, const float* __restrict__ Gt,
                                                    const int64_t* __restrict__ seqoff, const int32_t* __restrict__ cu,
                                                    const int2* __restrict__ sched, const int* __restrict__ count,
                                                    const float* __restrict__ gsc, float* __restrict__ dq,
                                                    float* __restrict__ dw) {
  constexpr int D = 128, BN = 64, R = 256 / HI;
  __shared__ __attribute__((aligned(16))) uint8_t t_lds[2][2][kKvTileB];
  const int n = blockIdx.x;
  if (n >= *count) return;
  const int2 e = sched[n];
  const int b = e.x;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int r0 = R * e.y, kend = min(L, r0 + R);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 31, hf = lane >> 5;
  const int v = 32 * w + qc;
  const int my_t = r0 + v / HI, head = v % HI;
  const bool valid = my_t < kend;
  const int trow = min(my_t, kend - 1);
  const int wave_tmax = min(kend - 1, r0 + (32 * w + 31) / HI);
  i32x4 qf[8];
  {
    const uint8_t* qp = q_idx + ((seq0 + trow) * HI + head) * D + 8 * hf;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) qf[s2] = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(qp + 16 * s2));
  }
  const float wq = wgt[(seq0 + trow) * HI + head];
  const float wqs = wq * gsc[0], unscale = gsc[1];
  const float* grow = tri_row(Gt, seqoff[b], trow);
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
  fp8_tile_store(t_lds[0][0], t_lds[0][1], pre, tid);
  __syncthreads();
  int buf = 0;
  for (int kt = 0; kt < kend; kt += BN) {
    const bool more = kt + BN < kend;
    if (more) gload(kt + BN);
    if (kt <= wave_tmax) {
      float gz[2][16];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
        const int key = 32 * rb + kperm(qc);
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          sacc = mfma_bf16_32x32x16(*reinterpret_cast<const i32x4*>(&t_lds[buf][0][kv_off(key, 32 * s2 + 16 * hf)]),
                                    qf[s2], sacc);
        // registers 4a .. 4a+3 <-> keys k0 .. k0+3 (consecutive)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int k0 = kt + 32 * rb + kperm(8 * a + 4 * hf);
          f32x4 g4 = {0.f, 0.f, 0.f, 0.f};
          if (valid && k0 <= my_t) g4 = *reinterpret_cast<const f32x4*>(grow + k0);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float s = sacc[4 * a + c];
            const bool on = valid && (k0 + c <= my_t) && s > 0.f;
            gz[rb][4 * a + c] = on ? g4[c] * wqs : 0.f;
            dwacc += on ? g4[c] * s : 0.f;
          }
        }
      }
      accumulate_xt_gt(t_lds[buf][1], gz, lane, o);
    }
    if (more) fp8_tile_store(t_lds[buf ^ 1][0], t_lds[buf ^ 1][1], pre, tid);
    __syncthreads();
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
          (f32x4){o[db][4 * a] * unscale, o[db][4 * a + 1] * unscale, o[db][4 * a + 2] * unscale,
                  o[db][4 * a + 3] * unscale};
}

// ------------------------------------------------------------------------------------------
// kl_dk_kernel<HI>: grid (256-key blocks, query-row slices of kDkSlice rows), 8 waves; lane
// column = key s = s0 + 32 wave + c; tiles of 64 consecutive (row, head) vectors of the slice.
// Writes partial dk [slice][T][128].
// ------------------------------------------------------------------------------------------
constexpr int kDkSlice = 1024;

template <int HI>
__global__ __launch_bounds__(512) void kl_dk_kernel(const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx,
                                                    const float* __restrict__ wgt, const float* __restrict__ Gt,
                                                    const int64_t* __restrict__ seqoff, const int32_t* __restrict__ cu,
                                                    const int2* __restrict__ sched, const int* __restrict__ count,
                                                    int64_t T, const float* __restrict__ gsc,
                                                    float* __restrict__ dk_part) {
  constexpr int D = 128, BN = 64, RPT = BN / HI;  // rows per tile
  __shared__ __attribute__((aligned(16))) uint8_t t_lds[2][2][kKvTileB];
  __shared__ float w_lds[2][BN];
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
  const float gs = gsc[0], unscale = gsc[1];
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  if (t_lo < t_hi) {
    i32x4 kf[8];
    {
      const uint8_t* kp = k_idx + (seq0 + srow) * D + 8 * hf;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) kf[s2] = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(kp + 16 * s2));
    }
    const int64_t v_begin = (int64_t)t_lo * HI, v_end = (int64_t)t_hi * HI;  // vectors of this slice
    uint4 pre;
    float wpre = 0.f;
    auto gload = [&](int64_t v0) {
      const int64_t vv = min(v0 + (tid >> 3), v_end - 1);
      pre = *reinterpret_cast<const uint4*>(q_idx + (seq0 * HI + vv) * D + 16 * (tid & 7));
      if (tid < BN) wpre = wgt[seq0 * HI + min(v0 + tid, v_end - 1)];
    };
    auto lstore = [&](int buf) {
      fp8_tile_store(t_lds[buf][0], t_lds[buf][1], pre, tid);
      if (tid < BN) w_lds[buf][tid] = wpre;
    };
    gload(v_begin);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int64_t v0 = v_begin; v0 < v_end; v0 += BN) {
      const bool more = v0 + BN < v_end;
      if (more) gload(v0 + BN);
      const int tt0 = int(v0 / HI);  // first row of the tile
      if (tt0 + RPT - 1 >= s0 + 32 * w) {  // some row of the tile sees some key of this wave
        // g[t, s] for the tile's rows (s <= t)
        float gr[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          const int tr = tt0 + r;
          gr[r] = (valid && tr < t_hi && my_s <= tr) ? tri_row(Gt, seqoff[b], tr)[my_s] : 0.f;
        }
        float gz[2][16];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x16 sacc;
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
          const int vrow = 32 * rb + kperm(qc);
#pragma unroll
          for (int s2 = 0; s2 < 8; ++s2)
            sacc = mfma_bf16_32x32x16(
                *reinterpret_cast<const i32x4*>(&t_lds[buf][0][kv_off(vrow, 32 * s2 + 16 * hf)]), kf[s2], sacc);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int vl = 32 * rb + kperm(8 * (i >> 2) + 4 * hf + (i & 3));  // vector within the tile
            const int r = vl / HI;
            const float gv = gr[r];
            const float s = sacc[i];
            gz[rb][i] = (s > 0.f) ? gv * (w_lds[buf][vl] * gs) : 0.f;
          }
        }
        accumulate_xt_gt(t_lds[buf][1], gz, lane, o);
      }
      if (more) lstore(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
  if (!valid) return;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<f32x4*>(op + 32 * db + 8 * a + 4 * hf) =
          (f32x4){o[db][4 * a] * unscale, o[db][4 * a + 1] * unscale, o[db][4 * a + 2] * unscale,
                  o[db][4 * a + 3] * unscale};
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
  const dim3 grid(nb128, (max_len + kKlTargetChunk - 1) / kKlTargetChunk);
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

hipError_t launch_kl_gscale(const float* w, int64_t n, float* part, float* gsc, hipStream_t st) {
  kl_wmax_kernel<<<kGscaleBlocks, 256, 0, st>>>(w, n, part);
  kl_gscale_kernel<<<1, 256, 0, st>>>(part, gsc);
  return hipGetLastError();
}

hipError_t launch_kl_dq(int H, const uint8_t* q_idx, const uint8_t* k_idx, const float* w, const float* G,
                        const int64_t* seqoff, const int32_t* cu, const int2* schedR, const int* countR, int nbR,
                        const float* gsc, float* dq, float* dw, hipStream_t st) {
  if (nbR == 0) return hipSuccess;
  switch (H) {
    case 16: kl_dq_kernel<16><<<nbR, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, schedR, countR, gsc, dq, dw); break;
    case 32: kl_dq_kernel<32><<<nbR, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, schedR, countR, gsc, dq, dw); break;
    case 64: kl_dq_kernel<64><<<nbR, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, schedR, countR, gsc, dq, dw); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int kl_dk_slices(int max_len) { return (max_len + kDkSlice - 1) / kDkSlice; }

hipError_t launch_kl_dk(int H, const uint8_t* q_idx, const uint8_t* k_idx, const float* w, const float* G,
                        const int64_t* seqoff, const int32_t* cu, int nseq, const int2* sched256,
                        const int* count256, int nb256, int max_len, int64_t T, const float* gsc, float* dk_part,
                        float* dk, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid(nb256, kl_dk_slices(max_len));
  switch (H) {
    case 16: kl_dk_kernel<16><<<grid, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, sched256, count256, T, gsc, dk_part); break;
    case 32: kl_dk_kernel<32><<<grid, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, sched256, count256, T, gsc, dk_part); break;
    case 64: kl_dk_kernel<64><<<grid, 512, 0, st>>>(q_idx, k_idx, w, G, seqoff, cu, sched256, count256, T, gsc, dk_part); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  kl_dk_reduce_kernel<<<(unsigned)T, 128, 0, st>>>(dk_part, cu, nseq, T, dk);
  return hipGetLastError();
}

}  // namespace dsa
