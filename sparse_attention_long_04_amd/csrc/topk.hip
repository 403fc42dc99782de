// Deterministic per-row top-k over indexer scores (Keye-VL-2.0 summary page, gsyq.cn,
// section 一: keep the k most relevant positions per token; section 八: the selection must
// be deterministic so that training and inference agree).
//
// Rule: the first min(k, n) keys in the order (score descending, index ascending), written in
// ascending index order and padded with -1.
//
// One workgroup (256 threads) per row.  Scores are mapped to order-preserving uint32 keys and
// the k-th largest key T is found by a most-significant-digit radix select (digits of 12, 12
// and 8 bits, histograms in LDS).  Then one ordered stream compaction keeps every key > T and
// the lowest-index keys == T until k are kept; a block-wide prefix sum gives each kept key its
// output slot, so the output comes out sorted with no sort pass.
#include "common.h"

namespace dsa {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / 64;

struct TopkSmem {
  int hist[4096];
  int wave_tot[kTopkWaves];
  int sel_digit;
  int sel_above;
};

// Block-wide inclusive scan (256 threads).  Returns the inclusive prefix, *total = block sum.
__device__ __forceinline__ int block_incl_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = wave_incl_scan(v);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int t = wave_tot[w];
    if (w < wave) before += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return incl + before;
}

__device__ void select_row(const float* __restrict__ row, int n, int K, int32_t* __restrict__ out,
                           TopkSmem& sm) {
  const int tid = threadIdx.x;
  if (n <= K) {
    for (int s = tid; s < K; s += kTopkThreads) out[s] = (s < n) ? s : -1;
    return;
  }
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  uint32_t prefix = 0, hi_mask = 0;
  int krem = K;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int d = 0; d < 3; ++d) {
    const int shift = shifts[d];
    const int nb = 1 << widths[d];
    const uint32_t dmask = uint32_t(nb - 1);
    for (int i = tid; i < nb; i += kTopkThreads) sm.hist[i] = 0;
    __syncthreads();
    if (aligned) {
      const int n4 = n >> 2;
      for (int q = tid; q < n4; q += kTopkThreads) {
        const f32x4 v = reinterpret_cast<const f32x4*>(row)[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = score_key(v[e]);
          if ((key & hi_mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & dmask], 1);
        }
      }
      for (int s = (n4 << 2) + tid; s < n; s += kTopkThreads) {
        const uint32_t key = score_key(row[s]);
        if ((key & hi_mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & dmask], 1);
      }
    } else {
      for (int s = tid; s < n; s += kTopkThreads) {
        const uint32_t key = score_key(row[s]);
        if ((key & hi_mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & dmask], 1);
      }
    }
    __syncthreads();
    // thread tid owns bins [nb - bpt*(tid+1), nb - bpt*tid), scanned from the top
    const int bpt = nb / kTopkThreads;
    const int top = nb - bpt * tid;
    int local = 0;
    for (int i = 1; i <= bpt; ++i) local += sm.hist[top - i];
    int total;
    const int incl = block_incl_scan(local, sm.wave_tot, &total);
    const int excl = incl - local;
    if (excl < krem && krem <= incl) {
      int c = excl;
      for (int i = 1; i <= bpt; ++i) {
        const int h = sm.hist[top - i];
        if (c + h >= krem) {
          sm.sel_digit = top - i;
          sm.sel_above = c;
          break;
        }
        c += h;
      }
    }
    __syncthreads();
    const int digit = sm.sel_digit;
    krem -= sm.sel_above;
    prefix |= uint32_t(digit) << shift;
    hi_mask |= dmask << shift;
    __syncthreads();
  }
  // prefix = key of the k-th largest score; krem = how many keys equal to it are kept.
  const uint32_t T = prefix;
  int base_gt = 0, base_eq = 0;
  for (int c0 = 0; c0 < n; c0 += 4 * kTopkThreads) {
    const int s0 = c0 + 4 * tid;
    uint32_t keys[4];
    if (aligned && s0 + 3 < n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + s0);
#pragma unroll
      for (int e = 0; e < 4; ++e) keys[e] = score_key(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) keys[e] = (s0 + e < n) ? score_key(row[s0 + e]) : 0u;
    }
    int cgt = 0, ceq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool valid = s0 + e < n;
      cgt += (valid && keys[e] > T);
      ceq += (valid && keys[e] == T);
    }
    const int packed = cgt | (ceq << 16);
    int total;
    const int incl = block_incl_scan(packed, sm.wave_tot, &total);
    const int excl = incl - packed;
    int gt_before = base_gt + (excl & 0xFFFF);
    int eq_before = base_eq + (excl >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (s0 + e >= n) break;
      if (keys[e] > T) {
        out[gt_before + min(eq_before, krem)] = s0 + e;
        ++gt_before;
      } else if (keys[e] == T) {
        if (eq_before < krem) out[gt_before + eq_before] = s0 + e;
        ++eq_before;
      }
    }
    base_gt += total & 0xFFFF;
    base_eq += total >> 16;
  }
}

// Prefill rows: one workgroup per token, longest rows first (row t = T-1-blockIdx.x).
__global__ __launch_bounds__(kTopkThreads) void topk_prefill_kernel(
    const float* __restrict__ tri, const int64_t* __restrict__ seqoff, const int32_t* __restrict__ cu,
    int nseq, int64_t T, int K, int32_t* __restrict__ out) {
  __shared__ TopkSmem sm;
  const int64_t t = T - 1 - (int64_t)blockIdx.x;
  const int b = find_seq(cu, nseq, t);
  const int i = int(t - cu[b]);
  const int j = i >> 4;
  const float* row = tri + seqoff[b] + score_block_offset(j) + (i & 15) * 16 * (int64_t)(j + 1);
  select_row(row, i + 1, K, out + t * K, sm);
}

// Decode rows: one workgroup per sequence, n = cache_lens[b].
__global__ __launch_bounds__(kTopkThreads) void topk_decode_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ cache_lens, int K,
    int32_t* __restrict__ out) {
  __shared__ TopkSmem sm;
  const int b = blockIdx.x;
  select_row(scores + b * ld, cache_lens[b], K, out + (int64_t)b * K, sm);
}

hipError_t launch_topk_prefill(const float* tri, const int64_t* seqoff, const int32_t* cu, int nseq,
                               int64_t T, int K, int32_t* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  topk_prefill_kernel<<<(unsigned)T, kTopkThreads, 0, st>>>(tri, seqoff, cu, nseq, T, K, out);
  return hipGetLastError();
}

hipError_t launch_topk_decode(const float* scores, int64_t ld, const int32_t* cache_lens, int B, int K,
                              int32_t* out, hipStream_t st) {
  topk_decode_kernel<<<B, kTopkThreads, 0, st>>>(scores, ld, cache_lens, K, out);
  return hipGetLastError();
}

}  // namespace dsa
