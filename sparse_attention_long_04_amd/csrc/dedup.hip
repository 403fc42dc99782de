// Adjacent-query dedup for the sparse attention (Keye-VL-2.0 summary page, gsyq.cn, section 八:
// the top-k sets of adjacent query tokens overlap heavily, so a block of adjacent queries
// attends over the union of their sets once -- one MFMA tile per key tile of the union, with a
// per-(query, key) mask -- instead of gathering every query's keys separately).
//
// The result is the plain sparse attention over each row's own set: a masked-out key
// contributes exp(-inf) = 0 to the row's softmax, so only the order of the fp32 sums differs.
//
// union_kernel -- one workgroup per block of kDedupRows = 16 adjacent rows of one sequence
//   (16-row blocks, longest first).  The block's key range [0, last row] is swept in chunks of
//   kUnionChunk positions: each row's sorted index list is cut at the chunk end by a binary
//   search, its keys set the row's bit in an LDS mask array (integer atomicOr, two 16-bit masks
//   per word, padded one word in 33 against bank conflicts), and an ordered block-wide
//   compaction appends every (key, mask) with a non-zero mask.  Output: the union in ascending
//   key order, one 16-bit row mask per key, and its size.
//
// dedup_attention_kernel -- one workgroup per (16-row block, KV head g); its G/2 waves hold the
//   block's 16 x G query vectors of group g, 32 per wave (row (32w + c) / G, head g G +
//   (32w + c) % G for lane column c).  The union is swept in 64-key tiles: K and V rows of head g
//   gathered from HBM into registers, then written to a double-buffered LDS tile (V as fp16);
//   S^T = K Q^T with bf16 32x32x16 MFMAs, the mask applied per element, online softmax in
//   fp32, O^T += V^T P^T with fp16 MFMAs whose V^T operand is read transposed from LDS.  Each
//   wave turns the tile's 64 row masks into one 64-bit key mask per row with ballots.  The
//   workgroup index maps to (block, head) with the head = index mod Hkv, so (the dispatcher
//   dealing workgroups round-robin over the 8 XCDs) every XCD gathers a single head's rows.
#include "attn_tiles.h"

namespace dsa {

constexpr int kDedupRows = 16;
constexpr int kUnionChunk = 16384;                       // key positions per LDS sweep
constexpr int kUnionWords = kUnionChunk / 2;             // two 16-bit masks per word
constexpr int kUnionWordsPadded = kUnionWords + kUnionWords / 32;

__device__ __forceinline__ int union_word(int w) { return w + (w >> 5); }

__global__ __launch_bounds__(256) void union_kernel(const int32_t* __restrict__ idx, int K,
                                                    const int32_t* __restrict__ cu, const int2* __restrict__ sched,
                                                    const int* __restrict__ sched_count, int64_t ustride,
                                                    int32_t* __restrict__ ukeys, uint16_t* __restrict__ umask,
                                                    int* __restrict__ ucount) {
  __shared__ uint32_t wmask[kUnionWordsPadded];
  __shared__ int rbeg[kDedupRows], rend[kDedupRows];
  __shared__ int wave_tot[4];
  const int n = blockIdx.x;
  if (n >= *sched_count) return;
  const int2 e = sched[n];
  const int b = e.x, j = e.y;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int i0 = kDedupRows * j;
  const int nr = min(kDedupRows, L - i0);
  const int plast = i0 + nr - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* __restrict__ uk = ukeys + (int64_t)n * ustride;
  uint16_t* __restrict__ um = umask + (int64_t)n * ustride;
  if (tid < kDedupRows) rbeg[tid] = 0;
  int base = 0;
  for (int c0 = 0; c0 <= plast; c0 += kUnionChunk) {
    const int c1 = c0 + kUnionChunk;
    for (int i = tid; i < kUnionWordsPadded; i += 256) wmask[i] = 0u;
    if (tid < nr) {
      // first entry >= c1 in row tid's ascending list of min(K, i+1) keys
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
      for (int x = rbeg[r] + tid; x < rend[r]; x += 256) {
        const int key = row[x] - c0;
        atomicOr(&wmask[union_word(key >> 1)], (1u << r) << (16 * (key & 1)));
      }
    }
    __syncthreads();
    // ordered compaction: thread tid owns words 32 tid .. 32 tid + 31 (keys c0 + 64 tid ...)
    int cnt = 0;
    for (int w = 0; w < 32; ++w) {
      const uint32_t x = wmask[union_word(32 * tid + w)];
      cnt += ((x & 0xFFFFu) != 0u) + ((x >> 16) != 0u);
    }
    int incl = wave_incl_scan(cnt);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      before += (w < wave) ? wave_tot[w] : 0;
      total += wave_tot[w];
    }
    int pos = base + before + incl - cnt;
    for (int w = 0; w < 32; ++w) {
      const uint32_t x = wmask[union_word(32 * tid + w)];
      const int key = c0 + 64 * tid + 2 * w;
      if (x & 0xFFFFu) {
        uk[pos] = key;
        um[pos] = uint16_t(x & 0xFFFFu);
        ++pos;
      }
      if (x >> 16) {
        uk[pos] = key + 1;
        um[pos] = uint16_t(x >> 16);
        ++pos;
      }
    }
    base += total;
    if (tid < nr) rbeg[tid] = rend[tid];
    __syncthreads();
  }
  if (tid == 0) ucount[n] = base;
}

// Two waves per SIMD for groups of 8 and 16 query heads; smaller groups give each wave 8 or 16
// rows of softmax state, which only fits at one.
template <int G>
__global__ __launch_bounds__(32 * G) __attribute__((amdgpu_waves_per_eu(G >= 8 ? 2 : 1, 2))) void dedup_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu, int Hq, int Hkv, float scale_log2, const int2* __restrict__ sched,
    const int* __restrict__ sched_count, int64_t ustride, const int32_t* __restrict__ ukeys,
    const uint16_t* __restrict__ umask, const int* __restrict__ ucount, uint16_t* __restrict__ out) {
  constexpr int D = 128, BN = 64, NTH = 32 * G, UPT = 1024 / NTH;  // 16-byte units per thread
  constexpr int RW = 32 / G;                                       // rows per wave
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "a wave's 32 query vectors must span whole rows");
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2][2][kKvTileB];  // [buffer][K=0/V=1]
  const int n = blockIdx.x / Hkv;
  const int g = blockIdx.x % Hkv;
  if (n >= *sched_count) return;
  const int2 e = sched[n];
  const int b = e.x, j = e.y;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int i0 = kDedupRows * j;
  const int nr = min(kDedupRows, L - i0);
  const int U = ucount[n];
  const int32_t* __restrict__ uk = ukeys + (int64_t)n * ustride;
  const uint16_t* __restrict__ um = umask + (int64_t)n * ustride;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int qc = lane & 31, hf = lane >> 5;
  const int qv = 32 * w + qc;
  const int my_r = qv / G;                 // row of this lane's query vector
  const int head = g * G + qv % G;
  const int rbase = (32 * w) / G;          // first row held by this wave
  const int64_t kvs = (int64_t)Hkv * D;

  i32x4 qf[8];
  {
    const int rr = min(my_r, nr - 1);
    const uint16_t* qp = q + ((seq0 + i0 + rr) * Hq + head) * D + 8 * hf;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) qf[s2] = *reinterpret_cast<const i32x4*>(qp + 16 * s2);
  }
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;

  // tile loader: 64 union keys x 16 units of 16 B for K and for V.  The union positions of a
  // tile are read two tiles ahead into an LDS ring (upos), so the gathers never wait on them.
  __shared__ int upos[2][BN];
  i32x4 pre[2 * UPT];
  auto gload = [&](const int* pos) {
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int u = tid + NTH * x;  // unit: key = u >> 4, column = u & 15
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
      float vf[8];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) vf[e2] = bf16_to_f32(bf16_lane(pre[UPT + x], e2));
      *reinterpret_cast<i32x4*>(&kv_lds[buf][1][off]) = pack_f16x8(vf);
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
    const int pos2 = (tid < BN) ? uk[min(u0 + 2 * BN + tid, U - 1)] : 0;  // tile t + 2
    // this wave's rows: 64-bit key masks of the tile (bit = tile key), one per row, by ballot
    const int mk = (u0 + lane < U) ? int(um[u0 + lane]) : 0;
    uint64_t myword = 0;
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      const uint64_t bw = __ballot((mk >> (rbase + rr)) & 1);
      if (my_r == rbase + rr) myword = bw;
    }
    // register (i, rb) of this lane <-> bit c(i) of half rb of the shifted word
    const uint64_t mw = myword >> (8 * hf);
    const uint32_t mlo = uint32_t(mw), mhi = uint32_t(mw >> 32);
    const uint8_t* kl = kv_lds[buf][0];
    const uint8_t* vl = kv_lds[buf][1];
    f32x16 sacc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[rb][i] = 0.f;
      const int key = 32 * rb + kperm(qc);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2)
        sacc[rb] = mfma_bf16_32x32x16(*reinterpret_cast<const i32x4*>(kl + kv_off(key, 32 * s2 + 16 * hf)), qf[s2],
                                      sacc[rb]);
    }
    // C row (reg i, half hf) of block rb <-> tile key 32rb + kperm(8(i/4) + 4hf + i%4)
    //                                      = 32rb + 16(i/8) + 4((i/4)%2) + i%4 + 8hf
    float z[2][16];
    float mt = -__builtin_inff();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t bit = 1u << (16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3));
        const float zz = ((rb ? mhi : mlo) & bit) ? sacc[rb][i] : -__builtin_inff();
        z[rb][i] = zz;
        mt = fmaxf(mt, zz);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;  // unscaled max, then scaled (scale > 0)
    // lazy rescale: the reference max moves only when a lane's max passes it by more than
    // kLazy (log2 units), so p = 2^(s - ref) <= 2^kLazy and the O / sum rescale is rare
    constexpr float kLazy = 8.f;
    const bool upd = mt > m_run + kLazy;
    if (__any(upd)) {
      const float m_new = upd ? mt : m_run;
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;
    float ps = 0.f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(z[rb][i], scale_log2, -m_use));
        z[rb][i] = pv;
        ps += pv;
      }
    l_run += ps;
    const int grp = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        const i32x4 pf = pack_f16x8(&z[rb][8 * kk2]);
        const int key_a = 32 * rb + 16 * kk2 + 8 * (grp >> 1) + (jj >> 2);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int dim0 = 32 * db + 16 * (grp & 1) + 4 * (jj & 3);
          const s16x4 lo = lds_tr16(vl + kv_off(key_a, 2 * dim0));
          const s16x4 hi = lds_tr16(vl + kv_off(key_a + 4, 2 * dim0));
          const i32x4 a = __builtin_bit_cast(i32x4, (s16x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          o[db] = mfma_f16_32x32x16(a, pf, o[db]);
        }
      }
    if (more) lstore(buf ^ 1);
    if (tid < BN) upos[t & 1][tid] = pos2;  // tile t's slot: its gather was issued last iteration
    __syncthreads();
    buf ^= 1;
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_r >= nr) return;
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  uint16_t* op = out + ((seq0 + i0 + my_r) * Hq + head) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dim = 32 * db + 8 * a + 4 * hf;
      const uint32_t lo = f32_to_bf16(o[db][4 * a + 0] * inv) | (uint32_t(f32_to_bf16(o[db][4 * a + 1] * inv)) << 16);
      const uint32_t hi = f32_to_bf16(o[db][4 * a + 2] * inv) | (uint32_t(f32_to_bf16(o[db][4 * a + 3] * inv)) << 16);
      *reinterpret_cast<uint2*>(op + dim) = make_uint2(lo, hi);
    }
}

// ------------------------------------------------------------------------------------------
hipError_t launch_union(const int32_t* idx, int K, const int32_t* cu, const int2* sched, const int* count,
                        int nb_bound, int64_t ustride, int32_t* ukeys, uint16_t* umask, int* ucount, hipStream_t st) {
  if (nb_bound == 0) return hipSuccess;
  union_kernel<<<nb_bound, 256, 0, st>>>(idx, K, cu, sched, count, ustride, ukeys, umask, ucount);
  return hipGetLastError();
}

hipError_t launch_dedup_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu, int Hq,
                                  int Hkv, float scale, const int2* sched, const int* count, int nb_bound,
                                  int64_t ustride, const int32_t* ukeys, const uint16_t* umask, const int* ucount,
                                  uint16_t* out, hipStream_t st) {
  if (nb_bound == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  const unsigned grid = (unsigned)(nb_bound * Hkv);
  switch (Hq / Hkv) {
#define DSA_DEDUP(GG)                                                                                            \
  case GG:                                                                                                      \
    dedup_attention_kernel<GG><<<grid, 32 * GG, 0, st>>>(q, k, v, cu, Hq, Hkv, sl2, sched, count, ustride, ukeys, \
                                                         umask, ucount, out);                                   \
    break;
    DSA_DEDUP(2)
    DSA_DEDUP(4)
    DSA_DEDUP(8)
    DSA_DEDUP(16)
#undef DSA_DEDUP
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa
