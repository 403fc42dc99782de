// Row order for the prefill sparse-attention gather.
//
// Every row (query token) of the gather reads the K/V rows of its own k selected keys; the
// kernel's L2 and the memory-side cache only help when the rows in flight at once select the
// same keys.  With the index sets in hand (after the top-k), rows are therefore taken in the
// order of the key block that most of their selection falls in ("dominant block", 1024 keys
// when the sequences allow): rows whose selections concentrate in the same part of the
// context run together and share those keys' lines.  The order changes nothing else -- every
// row is computed on its own and written to its own output row.
//
// For long contexts (a sequence of 64K tokens or more) the key is two-level: the two blocks
// holding most of the row's selection, as an unordered pair (the lower block, then the higher
// one in up to 128 buckets), so that rows taken together share their two busiest stretches of
// keys.
//
// A counting sort of the rows by that key, with no global atomics (neighbouring rows rarely
// share a key, and device-wide atomics on a few hundred counters serialise):
//   row_signature_kernel  one wave per row (four consecutive rows per wave): LDS histogram of
//                         its selected positions >> shift, the fullest bin and the next
//                         fullest (lowest on ties; the fullest again when no other bin is
//                         used), key = (global block of the lower) * 2^sub_bits + the higher
//                         one's bucket
//   row_order_count       one workgroup per chunk of rows: LDS count per key, written out as
//                         the chunk's row of a [chunk][key] matrix
//   row_order_colscan    one thread per key: each (chunk, key) entry becomes the key's rows in
//                         the chunks before, and the key's total goes to a row after the matrix
//   row_order_keyscan    one workgroup: the totals become each key's first slot (keys
//                         ascending, chunks ascending inside a key)
//   row_order_scatter     one workgroup per chunk: each row takes the next slot of its
//                         (chunk, key) through an LDS atomic (the order inside a chunk and key
//                         is unspecified, which the results do not depend on)
#include "common.h"

namespace dsa {

constexpr int kSigBins = 1024;          // histogram bins per row (4 KiB of LDS per wave)
constexpr int kSigRowsPerWave = 4;      // consecutive rows per wave of the signature kernel
constexpr int kOrderMaxKeys = 32768;    // LDS counters per chunk (128 KiB); beyond: identity order
constexpr int kSigSubBitsMax = 7;       // second-level buckets per dominant block: up to 128
constexpr int kSigSubMinSeq = 65536;    // longest sequence below this: first level only
constexpr int kOrderCountMax = 1 << 20; // [chunk][key] matrix entries (4 MiB of workspace)
constexpr int kOrderMaxChunks = 1024;
constexpr int kOrderMinRows = 4096;     // rows per chunk at least
constexpr int kOrderThreads = 1024;

struct OrderPlan {
  int shift = 0, sub_bits = 0, sub_shift = 0, nkeys = 0, chunks = 0;
  int64_t rows = 0;  // rows per chunk
};

// Block size 2^shift (1024 keys or coarser, so that every row fits kSigBins bins and the
// first-level key space stays below kOrderMaxKeys / 2), the second level's 2^sub_bits buckets
// (a sequence's block b falls in bucket b >> sub_shift; as many buckets as blocks when the key
// space allows, at most 2^kSigSubBitsMax) and the chunking of the rows; nkeys = 0: no
// reordering.
static OrderPlan order_plan(int64_t T, int max_seqlen, int nseq) {
  OrderPlan p;
  int shift = 10;
  while ((int64_t(max_seqlen) >> shift) >= kSigBins) ++shift;
  while ((T >> shift) >= kOrderMaxKeys / 2) ++shift;
  const int64_t nblk = (T >> shift) + nseq + 2;  // first-level keys
  int seq_bits = 0;  // a row's blocks: 0 .. (max_seqlen - 1) >> shift, below 2^seq_bits
  while ((int64_t(1) << seq_bits) < ((int64_t(max_seqlen - 1) >> shift) + 1)) ++seq_bits;
  // measured (attention ms, first level only -> with the second): 128K 35.4 -> 30.7, the 256K
  // batch of six (longest 81K) 55.8 -> 51.4, but 32K 5.9 -> 6.1 .. 7.3 (2 .. 5 bits): short
  // contexts keep the first level alone
  int sub_bits = max_seqlen >= kSigSubMinSeq ? std::min(kSigSubBitsMax, seq_bits) : 0;
  while (sub_bits > 0 && (nblk << sub_bits) > kOrderMaxKeys) --sub_bits;
  const int64_t nkeys = nblk << sub_bits;
  if (T <= 0 || nkeys > kOrderMaxKeys) return p;
  p.sub_bits = sub_bits;
  p.sub_shift = seq_bits - sub_bits;
  const int64_t gmax = std::min<int64_t>(kOrderMaxChunks, kOrderCountMax / nkeys);
  p.shift = shift;
  p.nkeys = int(nkeys);
  p.rows = std::max<int64_t>(kOrderMinRows, (T + gmax - 1) / gmax);
  p.chunks = int((T + p.rows - 1) / p.rows);
  return p;
}

// Ints the ordering needs in the workspace: the [chunk][key] matrix and one row of key totals;
// 0 = no reordering.
int64_t row_order_count_ints(int64_t T, int max_seqlen, int nseq) {
  const OrderPlan p = order_plan(T, max_seqlen, nseq);
  return int64_t(p.chunks + 1) * p.nkeys;
}

__global__ __launch_bounds__(256) void row_signature_kernel(const int32_t* __restrict__ idx, int K,
                                                            const int32_t* __restrict__ cu, int nseq, int64_t T,
                                                            int shift, int sub_bits, int sub_shift,
                                                            int* __restrict__ sig) {
  __shared__ int hist[4][kSigBins];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t0 = ((int64_t)blockIdx.x * 4 + w) * kSigRowsPerWave;
  if (t0 >= T) return;  // waves are independent: no workgroup barrier below
  int* h = hist[w];
  for (int r = 0; r < kSigRowsPerWave && t0 + r < T; ++r) {
    const int64_t t = t0 + r;
    const int b = find_seq(cu, nseq, t);
    const int i = int(t - cu[b]);
    const int nb = (i >> shift) + 1;  // <= kSigBins by the choice of shift
    const int m = min(K, i + 1);      // the row's selected positions, all in [0, i]
    for (int x = lane; x < nb; x += 64) h[x] = 0;
    __builtin_amdgcn_wave_barrier();  // the wave's own LDS operations are performed in order
    // A chunk is 2048 positions: load u of the wave reads 1 KiB at once, lane l positions
    // 256u + 4l .. +3.  The row is ascending, so so are a lane's 32 values (in u, then in the
    // four), and runs of equal bins are added with one atomic each (one or two per lane).
    constexpr int CH = 8;
    const int32_t* row = idx + t * K;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    for (int j0 = 0; j0 < m; j0 += CH * 256) {
      int v[4 * CH];
      if (aligned && j0 + CH * 256 <= m) {
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          const i32x4 x = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(row + j0) + u * 64 + lane);
          v[4 * u] = x[0];
          v[4 * u + 1] = x[1];
          v[4 * u + 2] = x[2];
          v[4 * u + 3] = x[3];
        }
      } else {
#pragma unroll
        for (int u = 0; u < CH; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = j0 + (u * 64 + lane) * 4 + c;
            v[4 * u + c] = e < m ? row[e] : -1;
          }
      }
      int cur = -1, c = 0;
#pragma unroll
      for (int u = 0; u < 4 * CH; ++u) {
        const int bin = v[u] >= 0 ? min(v[u] >> shift, nb - 1) : -1;  // positions are <= i
        if (bin != cur) {
          if (c > 0) atomicAdd(&h[cur], c);
          cur = bin;
          c = 0;
        }
        c += bin >= 0;
      }
      if (c > 0) atomicAdd(&h[cur], c);
    }
    __builtin_amdgcn_wave_barrier();
    int best_c = -1, best_b = 0;
    for (int x = lane; x < nb; x += 64) {
      const int c = h[x];
      if (c > best_c) {  // ascending x: the lowest bin wins ties within a lane
        best_c = c;
        best_b = x;
      }
    }
    auto wave_best = [&](int& c, int& bb) {  // highest count, lowest bin on ties
      for (int o = 32; o > 0; o >>= 1) {
        const int oc = __shfl_xor(c, o), ob = __shfl_xor(bb, o);
        if (oc > c || (oc == c && ob < bb)) {
          c = oc;
          bb = ob;
        }
      }
    };
    wave_best(best_c, best_b);
    // the next fullest bin: the first one's count taken out by the lane that holds it
    __builtin_amdgcn_wave_barrier();
    if (lane == (best_b & 63)) h[best_b] = -1;
    __builtin_amdgcn_wave_barrier();
    int sec_c = -1, sec_b = 0;
    for (int x = lane; x < nb; x += 64) {
      const int c = h[x];
      if (c > sec_c) {
        sec_c = c;
        sec_b = x;
      }
    }
    wave_best(sec_c, sec_b);
    if (sec_c <= 0) sec_b = best_b;   // the whole selection in one block
    __builtin_amdgcn_wave_barrier();  // every lane has read h before the next row clears it
    // the two busiest blocks as an unordered pair: the lower one's global block, then the
    // higher one's bucket
    const int lo_b = min(best_b, sec_b), hi_b = max(best_b, sec_b);
    const int first = int((int64_t(cu[b]) + (int64_t(lo_b) << shift)) >> shift) + b;
    if (lane == 0) sig[t] = (first << sub_bits) | (hi_b >> sub_shift);
  }
}

// cnt[chunk * nkeys + key] = rows of the chunk with that key (every entry written).
__global__ __launch_bounds__(kOrderThreads) void row_order_count_kernel(const int* __restrict__ sig, int64_t T,
                                                                         int64_t rows, int nkeys,
                                                                         int* __restrict__ cnt) {
  __shared__ int h[kOrderMaxKeys];
  for (int x = threadIdx.x; x < nkeys; x += kOrderThreads) h[x] = 0;
  __syncthreads();
  const int64_t a = int64_t(blockIdx.x) * rows, e = std::min<int64_t>(T, a + rows);
  for (int64_t t = a + threadIdx.x; t < e; t += kOrderThreads) atomicAdd(&h[sig[t]], 1);
  __syncthreads();
  int* out = cnt + int64_t(blockIdx.x) * nkeys;
  for (int x = threadIdx.x; x < nkeys; x += kOrderThreads) out[x] = h[x];
}

// Column pass, one thread per key: cnt[g * nkeys + key] becomes the rows of that key in the
// chunks before g (in place), and tot[key] the key's rows over all chunks.  The chunks' counts
// are loaded kColBatch at a time before they are summed.
constexpr int kColBatch = 8;
__global__ __launch_bounds__(256) void row_order_colscan_kernel(int* __restrict__ cnt, int nkeys, int chunks,
                                                                 int* __restrict__ tot) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= nkeys) return;
  int run = 0;
  for (int g0 = 0; g0 < chunks; g0 += kColBatch) {
    int c[kColBatch];
#pragma unroll
    for (int u = 0; u < kColBatch; ++u) c[u] = g0 + u < chunks ? cnt[int64_t(g0 + u) * nkeys + x] : 0;
#pragma unroll
    for (int u = 0; u < kColBatch; ++u) {
      if (g0 + u < chunks) cnt[int64_t(g0 + u) * nkeys + x] = run;
      run += c[u];
    }
  }
  tot[x] = run;
}

// One workgroup: tot[key] becomes the first slot of the key (exclusive scan over the keys).
__global__ __launch_bounds__(kOrderThreads) void row_order_keyscan_kernel(int* __restrict__ tot, int nkeys) {
  __shared__ int part[kOrderThreads];
  const int tid = threadIdx.x;
  const int per = (nkeys + kOrderThreads - 1) / kOrderThreads;
  const int a = min(nkeys, tid * per), e = min(nkeys, a + per);
  int s = 0;
  for (int x = a; x < e; ++x) s += tot[x];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < kOrderThreads; o <<= 1) {  // inclusive scan of the per-thread sums
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int x = a; x < e; ++x) {
    const int c = tot[x];
    tot[x] = run;
    run += c;
  }
}

// Row t of chunk g takes slot keybase[key] + (rows of its key in earlier chunks) + its rank
// among the chunk's rows of that key (an LDS atomic).
__global__ __launch_bounds__(kOrderThreads) void row_order_scatter_kernel(const int* __restrict__ sig, int64_t T,
                                                                           int64_t rows, int nkeys,
                                                                           const int* __restrict__ first,
                                                                           const int* __restrict__ keybase,
                                                                           int32_t* __restrict__ order) {
  __shared__ int next[kOrderMaxKeys];
  const int* f = first + int64_t(blockIdx.x) * nkeys;
  for (int x = threadIdx.x; x < nkeys; x += kOrderThreads) next[x] = f[x] + keybase[x];
  __syncthreads();
  const int64_t a = int64_t(blockIdx.x) * rows, e = std::min<int64_t>(T, a + rows);
  for (int64_t t = a + threadIdx.x; t < e; t += kOrderThreads) order[atomicAdd(&next[sig[t]], 1)] = int32_t(t);
}

// Writes order[0..T) (a permutation of the rows).  cnt holds row_order_count_ints(...) ints.
// Returns hipErrorInvalidValue (nothing launched) when the key space is too large; the caller
// then keeps the identity order.
hipError_t launch_row_order(const int32_t* idx, int K, const int32_t* cu, int nseq, int64_t T, int max_seqlen,
                            int* sig, int* cnt, int32_t* order, hipStream_t st) {
  const OrderPlan p = order_plan(T, max_seqlen, nseq);
  if (p.nkeys == 0) return hipErrorInvalidValue;
  const int64_t per_block = 4 * kSigRowsPerWave;
  row_signature_kernel<<<(unsigned)((T + per_block - 1) / per_block), 256, 0, st>>>(idx, K, cu, nseq, T, p.shift,
                                                                                    p.sub_bits, p.sub_shift, sig);
  int* const tot = cnt + int64_t(p.chunks) * p.nkeys;  // the row after the matrix
  row_order_count_kernel<<<p.chunks, kOrderThreads, 0, st>>>(sig, T, p.rows, p.nkeys, cnt);
  row_order_colscan_kernel<<<(p.nkeys + 255) / 256, 256, 0, st>>>(cnt, p.nkeys, p.chunks, tot);
  row_order_keyscan_kernel<<<1, kOrderThreads, 0, st>>>(tot, p.nkeys);
  row_order_scatter_kernel<<<p.chunks, kOrderThreads, 0, st>>>(sig, T, p.rows, p.nkeys, cnt, tot, order);
  return hipGetLastError();
}

}  // namespace dsa
