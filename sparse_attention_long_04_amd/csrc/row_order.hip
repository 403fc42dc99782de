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
//   row_signature_kernel  one wave per row (four consecutive rows per wave): LDS histogram of
//                         its selected positions >> shift, the fullest bin (lowest on ties),
//                         key = global block of that bin; integer atomics count the rows per
//                         key, one per run of equal keys
//   row_order_scan_kernel one workgroup: exclusive prefix over the key counts
//   row_order_scatter     each row takes the next slot of its key (one atomic per run of equal
//                         keys in a wave; the order inside a key is unspecified, which the
//                         results do not depend on)
#include "common.h"

namespace dsa {

constexpr int kSigBins = 1024;       // histogram bins per row (4 KiB of LDS per wave)
constexpr int kOrderMaxKeys = 65536; // beyond this (very many sequences) the identity order is kept

// shift of the block size (1024 keys or coarser, so that every row fits kSigBins bins and the
// key space stays below kOrderMaxKeys); returns the number of keys, 0 = no reordering.
int row_order_keys(int64_t T, int max_seqlen, int nseq, int* shift_out) {
  int shift = 10;
  while ((int64_t(max_seqlen) >> shift) >= kSigBins) ++shift;
  while ((T >> shift) >= kOrderMaxKeys / 2) ++shift;
  const int64_t nkeys = (T >> shift) + nseq + 2;
  if (shift_out) *shift_out = shift;
  return nkeys <= kOrderMaxKeys ? int(nkeys) : 0;
}

__global__ __launch_bounds__(256) void row_order_clear_kernel(int* __restrict__ cnt, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) cnt[i] = 0;
}

constexpr int kSigRowsPerWave = 4;  // consecutive rows per wave: neighbours mostly share a key

__global__ __launch_bounds__(256) void row_signature_kernel(const int32_t* __restrict__ idx, int K,
                                                            const int32_t* __restrict__ cu, int nseq, int64_t T,
                                                            int shift, int* __restrict__ sig, int* __restrict__ cnt) {
  __shared__ int hist[4][kSigBins];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t0 = ((int64_t)blockIdx.x * 4 + w) * kSigRowsPerWave;
  if (t0 >= T) return;  // waves are independent: no workgroup barrier below
  int* h = hist[w];
  int run_key = -1, run_n = 0;  // lane 0: rows counted but not yet added to cnt
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
    for (int o = 32; o > 0; o >>= 1) {
      const int oc = __shfl_xor(best_c, o), ob = __shfl_xor(best_b, o);
      if (oc > best_c || (oc == best_c && ob < best_b)) {
        best_c = oc;
        best_b = ob;
      }
    }
    __builtin_amdgcn_wave_barrier();  // every lane has read h before the next row clears it
    if (lane == 0) {
      const int key = int((int64_t(cu[b]) + (int64_t(best_b) << shift)) >> shift) + b;
      sig[t] = key;
      if (key != run_key) {
        if (run_n > 0) atomicAdd(&cnt[run_key], run_n);
        run_key = key;
        run_n = 0;
      }
      ++run_n;
    }
  }
  if (lane == 0 && run_n > 0) atomicAdd(&cnt[run_key], run_n);
}

// Exclusive prefix over n counts in place (one workgroup of 1024 threads, n <= kOrderMaxKeys).
__global__ __launch_bounds__(1024) void row_order_scan_kernel(int* __restrict__ cnt, int n) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int a = min(n, tid * per), e = min(n, a + per);
  int s = 0;
  for (int x = a; x < e; ++x) s += cnt[x];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan of the 1024 partial sums
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int x = a; x < e; ++x) {
    const int c = cnt[x];
    cnt[x] = run;
    run += c;
  }
}

// Lanes of a wave whose keys equal their left neighbour's join its run: the run's first lane
// takes the run's slots with one atomic and each lane writes at its offset inside the run.
__global__ __launch_bounds__(256) void row_order_scatter_kernel(const int* __restrict__ sig, int64_t T,
                                                                int* __restrict__ off, int32_t* __restrict__ order) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const bool live = t < T;
  const int key = live ? sig[t] : -1;
  const int left = __shfl_up(key, 1);
  const uint64_t starts = __ballot(lane == 0 || key != left);
  const int lead = 63 - __builtin_clzll(starts & (~0ull >> (63 - lane)));  // this lane's run start
  const uint64_t after = lane < 63 ? starts & (~0ull << (lane + 1)) : 0ull;
  const int next = after ? __builtin_ctzll(after) : 64;  // first lane of the following run
  int base = 0;
  // rows past T hold key -1 and so start runs of their own: a live run holds live rows only
  if (lead == lane && live) base = atomicAdd(&off[key], next - lane);
  base = __shfl(base, lead);
  if (live) order[base + (lane - lead)] = int32_t(t);
}

// Writes order[0..T) (a permutation of the rows).  Returns hipErrorInvalidValue (nothing
// launched) when the key space is too large; the caller then keeps the identity order.
hipError_t launch_row_order(const int32_t* idx, int K, const int32_t* cu, int nseq, int64_t T, int max_seqlen,
                            int* sig, int* cnt, int32_t* order, hipStream_t st) {
  int shift = 0;
  const int nkeys = row_order_keys(T, max_seqlen, nseq, &shift);
  if (nkeys == 0 || T == 0) return hipErrorInvalidValue;
  row_order_clear_kernel<<<(nkeys + 255) / 256, 256, 0, st>>>(cnt, nkeys);
  row_signature_kernel<<<(unsigned)((T + 4 * kSigRowsPerWave - 1) / (4 * kSigRowsPerWave)), 256, 0, st>>>(idx, K, cu, nseq, T, shift, sig, cnt);
  row_order_scan_kernel<<<1, 1024, 0, st>>>(cnt, nkeys);
  row_order_scatter_kernel<<<(unsigned)((T + 255) / 256), 256, 0, st>>>(sig, T, cnt, order);
  return hipGetLastError();
}

}  // namespace dsa
