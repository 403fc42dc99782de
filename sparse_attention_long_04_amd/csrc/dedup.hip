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
//   (32w + c) % G for lane column c).  The union is swept in 64-key tiles: K (bf16) and V (an
//   fp16 copy) rows of head g copied straight from global memory into a double-buffered LDS
//   tile, the tile's union positions and row masks staged in LDS one tile ahead; S^T = K Q^T
//   with bf16 32x32x16 MFMAs, the mask applied per element, online softmax in fp32 with a lazy
//   reference maximum, O^T += V^T P^T with fp16 MFMAs whose V^T operand is read transposed from
//   LDS.  Per tile the work runs in four phases so that each half tile's softmax sits between
//   MFMAs: S(keys 0..31); S(32..63) beside softmax(0..31); O += (0..31) beside softmax(32..63);
//   O += (32..63).  Each wave turns the tile's 64 row masks into one 64-bit key mask per row
//   with ballots.  The workgroup index maps to (block, head) with the head = index mod Hkv, so
//   (the dispatcher dealing workgroups round-robin over the 8 XCDs) every XCD gathers a single
//   head's rows.
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
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vh,
    const int32_t* __restrict__ cu, int Hq, int Hkv, float scale_log2, const int2* __restrict__ sched,
    const int* __restrict__ sched_count, int64_t ustride, const int32_t* __restrict__ ukeys,
    const uint16_t* __restrict__ umask, const int* __restrict__ ucount, uint16_t* __restrict__ out) {
  constexpr int D = 128, BN = 64, NTH = 32 * G;
  constexpr int RW = 32 / G;  // rows per wave
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "a wave's 32 query vectors must span whole rows");
  __shared__ __attribute__((aligned(1024))) uint8_t kv_lds[2][2][kKvTileB];  // [buffer][K bf16 = 0 / V fp16 = 1]
  __shared__ int upos[2][BN], umk[2][BN];  // union positions and row masks of upcoming tiles
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
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) asm volatile("" : "+v"(qf[s2]));  // landed before any copy
  }
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16){};
  float m_run = -__builtin_inff(), l_run = 0.f;

  // K (bf16) and V (fp16) rows of the next tile, copied straight into LDS: copy x of this wave
  // fills rows 4 (CPW w + x) + lane/16 of the tile, LDS unit lane % 16 holding unit
  // (lane % 16) ^ s(row) (the kv_off swizzle); the positions come from upos.
  constexpr int CPW = 16 / (NTH / 64);  // 1 KB copies per wave and matrix
  lds_u8* const lb = (lds_u8*)&kv_lds[0][0][0];
  const uint32_t lds0 = (uint32_t)(uintptr_t)lb;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint16_t* const kg = k + seq0 * kvs + g * D;
  const uint16_t* const vg = vh + seq0 * kvs + g * D;
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
  constexpr float kLazy = 8.f;  // the reference max moves only when a row's max passes it by more
  const int grp = lane >> 4, jj = lane & 15;
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
    // this wave's rows: 64-bit key masks of the tile (bit = tile key), one per row, by ballot;
    // register (i, rb) of this lane <-> bit c(i) of half rb of the shifted word
    const int mk = umk[buf][lane];
    uint64_t myword = 0;
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      const uint64_t bw = __ballot((mk >> (rbase + rr)) & 1);
      if (my_r == rbase + rr) myword = bw;
    }
    const uint64_t mw = myword >> (8 * hf);
    const uint32_t mhalf[2] = {uint32_t(mw), uint32_t(mw >> 32)};
    const lds_u8* kl = lb + buf * 2 * kKvTileB;
    const lds_u8* vl = kl + kKvTileB;

    // S^T = K Q^T of keys 32 rb .. (8 MFMAs), C row (reg i, half hf) <-> tile key
    // 32 rb + 16(i/8) + 4((i/4)%2) + i%4 + 8 hf
    auto qk = [&](int rb, f32x16& s, auto&& between) {
      const int key = 32 * rb + kperm(qc);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        s = mfma_bf16_32x32x16(dn_ld128(kl + kv_off(key, 32 * s2 + 16 * hf)), qf[s2], s2 ? s : (f32x16){});
        between(s2);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // O^T += V^T P^T over keys 32 rb .. (8 MFMAs, V^T read transposed from LDS)
    auto pv = [&](int rb, const i32x4 (&pf)[2], auto&& between) {
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        const int key_a = 32 * rb + 16 * kk2 + 8 * (grp >> 1) + (jj >> 2);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int dim0 = 32 * db + 16 * (grp & 1) + 4 * (jj & 3);
          const s16x4 lo = lds_tr16_l(vl + kv_off(key_a, 2 * dim0));
          const s16x4 hi = lds_tr16_l(vl + kv_off(key_a + 4, 2 * dim0));
          const i32x4 a = __builtin_bit_cast(i32x4, (s16x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          o[db] = mfma_f16_32x32x16(a, pf[kk2], o[db]);
          between(4 * kk2 + db);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // softmax of half rb in two parts spread over 8 MFMA steps: steps 0-3 mask and maximum
    // (4 registers each), then the lazy reference check, steps 4-7 exponentials and packing.
    // Returns the rescale factor of O for this half (1 when the reference stayed).
    float z[16];
    i32x4 pf0[2], pf1[2];
    float alpha1 = 1.f;
    auto soft_mask = [&](const f32x16& s, uint32_t bits, int step, float& mt) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * step + c;
        const uint32_t bit = 1u << (16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3));
        const float zz = (bits & bit) ? s[i] : -__builtin_inff();
        z[i] = zz;
        mt = fmaxf(mt, zz);
      }
    };
    auto lazy = [&](float mt) -> float {  // returns alpha (1 if unchanged); updates m_run
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;
      const bool upd = mt > m_run + kLazy;
      float alpha = 1.f;
      if (__any(upd)) {
        const float m_new = upd ? mt : m_run;
        alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
      }
      return alpha;
    };
    auto soft_exp = [&](int step, i32x4 (&pf)[2], float& ps) {
      const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;
      float p[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        p[c] = __builtin_amdgcn_exp2f(fmaf(z[4 * step + c], scale_log2, -m_use));
        ps += p[c];
      }
      const f16x2 h01 = {(_Float16)p[0], (_Float16)p[1]}, h23 = {(_Float16)p[2], (_Float16)p[3]};
      int x01 = __builtin_bit_cast(int, h01), x23 = __builtin_bit_cast(int, h23);
      asm volatile("" : "+v"(x01), "+v"(x23));  // computed in this step
      pf[step >> 1][2 * (step & 1)] = x01;
      pf[step >> 1][2 * (step & 1) + 1] = x23;
    };

    // phase 1: S(keys 0..31)
    f32x16 s0, s1;
    qk(0, s0, [&](int) {});
    // phase 2: S(keys 32..63) beside the softmax of keys 0..31
    float mt0 = -__builtin_inff(), ps0 = 0.f;
    qk(1, s1, [&](int st) {
      if (st < 4) {
        soft_mask(s0, mhalf[0], st, mt0);
      } else {
        if (st == 4) {
          const float a0 = lazy(mt0);
          if (a0 != 1.f) {  // rare: rescale O and l now (keys 0..31 enter O next)
            l_run *= a0;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] *= a0;
          }
        }
        soft_exp(st - 4, pf0, ps0);
      }
    });
    l_run += ps0;
    // phase 3: O += keys 0..31 beside the softmax of keys 32..63
    float mt1 = -__builtin_inff(), ps1 = 0.f;
    pv(0, pf0, [&](int st) {
      if (st < 4) {
        soft_mask(s1, mhalf[1], st, mt1);
      } else {
        if (st == 4) alpha1 = lazy(mt1);
        soft_exp(st - 4, pf1, ps1);
      }
    });
    // phase 4: the rare rescale for keys 32..63 (after keys 0..31 entered O), then O += keys 32..63
    if (alpha1 != 1.f) {
      l_run *= alpha1;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha1;
    }
    l_run += ps1;
    pv(1, pf1, [&](int) {});
    if (tid < BN) {
      upos[buf][tid] = pos2;
      umk[buf ^ 1][tid] = mk1;
    }
    dn_sync();  // tile t+1 has landed; everyone is past tile t
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

hipError_t launch_dedup_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vh, const int32_t* cu, int Hq,
                                  int Hkv, float scale, const int2* sched, const int* count, int nb_bound,
                                  int64_t ustride, const int32_t* ukeys, const uint16_t* umask, const int* ucount,
                                  uint16_t* out, int max_len, hipStream_t st) {
  if (nb_bound == 0) return hipSuccess;
  // the K/V copy offsets are 32-bit byte offsets from the sequence's first row
  if (int64_t(max_len) * Hkv * 256 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  const float sl2 = scale * 1.4426950408889634f;
  const unsigned grid = (unsigned)(nb_bound * Hkv);
  switch (Hq / Hkv) {
#define DSA_DEDUP(GG)                                                                                            \
  case GG:                                                                                                      \
    dedup_attention_kernel<GG><<<grid, 32 * GG, 0, st>>>(q, k, vh, cu, Hq, Hkv, sl2, sched, count, ustride, ukeys, \
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
