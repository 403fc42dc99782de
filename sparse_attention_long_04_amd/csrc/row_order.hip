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
//   row_signature_kernel  one wave per row: LDS histogram of its selected positions >> shift,
//                         the fullest bin (lowest on ties), key = global block of that bin;
//                         integer atomics count the rows per key
//   row_order_scan_kernel one workgroup: exclusive prefix over the key counts
//   row_order_scatter     each row takes the next slot of its key (atomic; the order inside a
//                         key is unspecified, which the results do not depend on)
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

__global__ __launch_bounds__(256) void row_signature_kernel(const int32_t* __restrict__ idx, int K,
                                                            const int32_t* __restrict__ cu, int nseq, int64_t T,
                                                            int shift, int* __restrict__ sig, int* __restrict__ cnt) {
  __shared__ int hist[4][kSigBins];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + w;
  if (t >= T) return;  // waves are independent: no workgroup barrier below
  const int b = find_seq(cu, nseq, t);
  const int i = int(t - cu[b]);
  const int nb = (i >> shift) + 1;  // <= kSigBins by the choice of shift
  const int m = min(K, i + 1);      // the row's selected positions, all in [0, i]
  int* h = hist[w];
  for (int x = lane; x < nb; x += 64) h[x] = 0;
  __builtin_amdgcn_wave_barrier();  // the wave's own LDS operations are performed in order
  constexpr int RB = 8;             // index loads per lane issued together
  const int32_t* row = idx + t * K;
  for (int j0 = 0; j0 < m; j0 += RB * 64) {
    int v[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int j = j0 + u * 64 + lane;
      v[u] = j < m ? __builtin_nontemporal_load(row + j) : -1;
    }
#pragma unroll
    for (int u = 0; u < RB; ++u)
      if (v[u] >= 0) atomicAdd(&h[min(v[u] >> shift, nb - 1)], 1);  // positions are <= i
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
  if (lane == 0) {
    const int key = int((int64_t(cu[b]) + (int64_t(best_b) << shift)) >> shift) + b;
    sig[t] = key;
    atomicAdd(&cnt[key], 1);
  }
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

__global__ __launch_bounds__(256) void row_order_scatter_kernel(const int* __restrict__ sig, int64_t T,
                                                                int* __restrict__ off, int32_t* __restrict__ order) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  order[atomicAdd(&off[sig[t]], 1)] = int32_t(t);
}

// Writes order[0..T) (a permutation of the rows).  Returns hipErrorInvalidValue (nothing
// launched) when the key space is too large; the caller then keeps the identity order.
hipError_t launch_row_order(const int32_t* idx, int K, const int32_t* cu, int nseq, int64_t T, int max_seqlen,
                            int* sig, int* cnt, int32_t* order, hipStream_t st) {
  int shift = 0;
  const int nkeys = row_order_keys(T, max_seqlen, nseq, &shift);
  if (nkeys == 0 || T == 0) return hipErrorInvalidValue;
  row_order_clear_kernel<<<(nkeys + 255) / 256, 256, 0, st>>>(cnt, nkeys);
  row_signature_kernel<<<(unsigned)((T + 3) / 4), 256, 0, st>>>(idx, K, cu, nseq, T, shift, sig, cnt);
  row_order_scan_kernel<<<1, 1024, 0, st>>>(cnt, nkeys);
  row_order_scatter_kernel<<<(unsigned)((T + 255) / 256), 256, 0, st>>>(sig, T, cnt, order);
  return hipGetLastError();
}

}  // namespace dsa
