// Deterministic per-row top-k over indexer scores (Keye-VL-2.0 summary page, gsyq.cn,
// section 一: keep the k most relevant positions per token; section 八: the selection must
// be deterministic so that training and inference agree).
//
// Rule: the first min(k, n) keys in the order (score descending, index ascending), written in
// ascending index order and padded with -1.
//
// Scores map to order-preserving uint32 keys.  Scores of one row crowd into a few float
// exponents, so selection first bins them by VALUE: bin(x) = floor((x - lo) * nbins / (hi - lo))
// with the row's min lo and max hi (written by the indexer).  The map is monotone, so the
// threshold bin (the bin holding the k-th largest key) splits the row into elements that are
// surely kept (higher bins), surely dropped (lower bins) and the threshold bin's own elements,
// which are ranked exactly by (key descending, index ascending).  An ordered, block-wide prefix
// sum over the kept elements gives every one its output slot, so the output is sorted without
// a sort pass.  No float atomics anywhere; integer histogram atomics commute.
//
// Prefill (one workgroup per row, each of the 4 waves owning a contiguous quarter of the row):
// pass 1 builds per-wave histograms of 1024 value bins straight from HBM; pass 2 compacts every
// element whose bin is >= the threshold bin into an LDS list in index order (ballot + mbcnt
// inside the wave, per-wave offsets).  The threshold bin is then ranked pairwise when it holds
// at most 512 elements, else an exact most-significant-digit radix select (digits of 11, 11 and
// 10 bits) runs on the list.  Rows whose list would not fit in LDS (heavy ties) run the radix
// select over HBM; rows whose scores are all equal keep their first k keys directly.
//
// Decode rows (few rows of ~10^5 keys) are selected by decode_select.hip.
#include "common.h"

namespace dsa {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kListCap = 3072;     // LDS candidate list capacity (prefill)
constexpr int kBins = 2048;        // value bins / radix digit size

struct TopkSmem {
  int hist[kBins];
  int wave_tot[kTopkWaves];
  int sel_digit;
  int sel_above;
  int list_n;
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

// Given sm.hist[0..nb) filled, find the digit d with  above(d) < krem <= above(d) + hist[d],
// above(d) = sum of hist over digits > d.  Results in sm.sel_digit / sm.sel_above.
__device__ __forceinline__ void find_digit(TopkSmem& sm, int nb, int krem) {
  const int tid = threadIdx.x;
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
}

__device__ __forceinline__ void clear_hist(TopkSmem& sm, int nb) {
  for (int i = threadIdx.x; i < nb; i += kTopkThreads) sm.hist[i] = 0;
  __syncthreads();
}

// Monotone value bin of score x in a row with range [lo, lo + 1/sc].
__device__ __forceinline__ int value_bin(float x, float lo, float sc, int nbins = kBins) {
  return min(nbins - 1, int((x - lo) * sc));
}

__device__ __forceinline__ float key_to_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---- element sources: a raw score row (index = position) or a (key, index) list ----------
struct RowSrc {
  const float* __restrict__ row;
  bool vec;  // 16-byte aligned
  // visit elements [c0 + 4*tid, +4) of a 1024-element chunk in index order
  __device__ __forceinline__ void quad(int n, int s0, uint32_t* keys, int* ids) const {
    if (vec && s0 + 3 < n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + s0);
#pragma unroll
      for (int e = 0; e < 4; ++e) keys[e] = score_key(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) keys[e] = (s0 + e < n) ? score_key(row[s0 + e]) : 0u;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ids[e] = s0 + e;
  }
};

struct ListSrc {
  const uint32_t* __restrict__ keys;
  const int* __restrict__ ids;
  __device__ __forceinline__ void quad(int n, int s0, uint32_t* k, int* id) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = s0 + e < n;
      k[e] = ok ? keys[s0 + e] : 0u;
      id[e] = ok ? ids[s0 + e] : -1;
    }
  }
};

// Histogram of digit (key >> shift) & dmask over elements with (key & hmask) == prefix.
template <class Src>
__device__ void hist_pass(const Src& src, int n, uint32_t prefix, uint32_t hmask, int shift, uint32_t dmask,
                          TopkSmem& sm) {
  for (int c0 = 0; c0 < n; c0 += 4 * kTopkThreads) {
    uint32_t k[4];
    int id[4];
    const int s0 = c0 + 4 * threadIdx.x;
    src.quad(n, s0, k, id);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (s0 + e < n && (k[e] & hmask) == prefix) atomicAdd(&sm.hist[(k[e] >> shift) & dmask], 1);
  }
  __syncthreads();
}

// Radix select digits [d0, 3) over src.  On entry prefix/hmask describe the already fixed high
// bits and krem the number still to take among matching elements.  On exit prefix = T (the
// k-th largest key) and krem = how many keys equal to T are kept.
template <class Src>
__device__ void radix_rest(const Src& src, int n, int d0, uint32_t& prefix, uint32_t& hmask, int& krem,
                           TopkSmem& sm) {
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int d = d0; d < 3; ++d) {
    const int nb = 1 << widths[d];
    const uint32_t dmask = uint32_t(nb - 1);
    clear_hist(sm, nb);
    hist_pass(src, n, prefix, hmask, shifts[d], dmask, sm);
    find_digit(sm, nb, krem);
    krem -= sm.sel_above;
    prefix |= uint32_t(sm.sel_digit) << shifts[d];
    hmask |= dmask << shifts[d];
    __syncthreads();
  }
}

// Ordered compaction: call emit(slot, key, id) for every element kept by keep(key) in index
// order; slot counts kept elements.  Elements with key == T are kept only while fewer than
// krem of them have been seen (lowest indices first); keys > T are always kept.
template <class Src, class Emit>
__device__ void ordered_emit(const Src& src, int n, uint32_t T, int krem, Emit emit, TopkSmem& sm) {
  int base_gt = 0, base_eq = 0;
  for (int c0 = 0; c0 < n; c0 += 4 * kTopkThreads) {
    uint32_t k[4];
    int id[4];
    const int s0 = c0 + 4 * threadIdx.x;
    src.quad(n, s0, k, id);
    int cgt = 0, ceq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = s0 + e < n;
      cgt += (ok && k[e] > T);
      ceq += (ok && k[e] == T);
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
      if (k[e] > T) {
        emit(gt_before + min(eq_before, krem), k[e], id[e]);
        ++gt_before;
      } else if (k[e] == T) {
        if (eq_before < krem) emit(gt_before + eq_before, k[e], id[e]);
        ++eq_before;
      }
    }
    base_gt += total & 0xFFFF;
    base_eq += total >> 16;
  }
  __syncthreads();
}

// ---- finishing a candidate list ------------------------------------------------------------
// The list (keys, ids) holds, in index order, every element whose value bin is >= b1.  All of
// bin > b1 is kept; of the m elements in bin b1 the krem best under (key desc, id asc) are kept.
// They are ranked directly (m^2/256 comparisons per thread) and the dropped ones get key 0,
// which no score maps to; the output is then an ordered compaction of the non-zero keys.
template <int CAP>
struct FinishSmem {
  uint32_t sk[CAP];
  int sid[CAP];
  int spos[CAP];
  int sub_n;
};

// Returns false (list untouched) when bin b1 holds more than CAP elements.
template <int CAP, class BinOf>
__device__ __forceinline__ bool rank_threshold_bin(uint32_t* keys, const int* ids, int total, int b1, int krem, BinOf bin_of,
                                   FinishSmem<CAP>& fs) {
  constexpr int kSubCap = CAP;
  if (threadIdx.x == 0) fs.sub_n = 0;
  __syncthreads();
  // four list reads per wait (reads past the list are clamped to its last entry, then ignored)
  for (int i0 = threadIdx.x; i0 < total; i0 += 4 * kTopkThreads) {
    uint32_t kq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kq[u] = keys[min(i0 + u * kTopkThreads, total - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kTopkThreads;
      if (i < total && bin_of(kq[u]) == b1) {
        const int j = atomicAdd(&fs.sub_n, 1);
        if (j < kSubCap) {
          fs.sk[j] = kq[u];
          fs.sid[j] = ids[i];
          fs.spos[j] = i;
        }
      }
    }
  }
  __syncthreads();
  const int m = fs.sub_n;
  if (m > kSubCap) return false;
  for (int j = threadIdx.x; j < m; j += kTopkThreads) {
    const uint32_t k = fs.sk[j];
    const int id = fs.sid[j];
    int rank = 0;
#pragma unroll 8
    for (int x = 0; x < m; ++x) {
      const uint32_t kx = fs.sk[x];
      rank += (kx > k) | ((kx == k) & (fs.sid[x] < id));
    }
    if (rank >= krem) keys[fs.spos[j]] = 0u;
  }
  __syncthreads();
  return true;
}

// Ordered compaction of the list entries with a non-zero key, EPT entries per thread and round
// (each round is one block scan).
template <int EPT = 4>
__device__ void emit_nonzero(const uint32_t* keys, const int* ids, int total, int32_t* __restrict__ out,
                             TopkSmem& sm) {
  int base = 0;
  for (int c0 = 0; c0 < total; c0 += EPT * kTopkThreads) {
    const int s0 = c0 + EPT * threadIdx.x;
    bool keep[EPT];
    int c = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      keep[e] = (s0 + e < total) && keys[s0 + e] != 0u;
      c += keep[e];
    }
    int tot;
    const int incl = block_incl_scan(c, sm.wave_tot, &tot);
    int pos = base + incl - c;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (keep[e]) out[pos++] = ids[s0 + e];
    base += tot;
  }
  __syncthreads();
}

// ---- prefill row select: per-wave segments, no block barriers inside the two HBM passes ----
constexpr int kQ = 8;  // float4 loads in flight per lane per wave step (2048 elements)
constexpr int kVBins = 1024;  // value bins of the prefill pass 1 (per wave)

struct TopkRowSmem {
  TopkSmem s;
  union {
    int whist[kTopkWaves][kVBins];  // pass 1: per-wave value histograms
    struct {
      uint32_t lkeys[kListCap];    // pass 2 on: candidate list (index order)
      int lids[kListCap];
    } l;
  } u;
  int wcnt[kTopkWaves];
  int woff[kTopkWaves];
  FinishSmem<512> f;
};

__device__ __forceinline__ void first_k(int n, int K, int32_t* __restrict__ out) {
  for (int s = threadIdx.x; s < K; s += kTopkThreads) out[s] = (s < n) ? s : -1;
}

// Load the wave step [base, base + 1024) of a segment ending at hi: lane gets elements
// base + 4(lane + 64e) + j; slots past hi read as `fill` (callers either flag them invalid or
// fill -inf, which no threshold test passes).
__device__ __forceinline__ void load_step(const float* __restrict__ row, int base, int hi, int lane, f32x4 (&v)[kQ],
                                          float fill = 0.f) {
#pragma unroll
  for (int e = 0; e < kQ; ++e) {
    const int i = base + 4 * (lane + 64 * e);
    if (i + 3 < hi) {
      v[e] = *reinterpret_cast<const f32x4*>(row + i);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[e][j] = (i + j < hi) ? row[i + j] : fill;
    }
  }
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
}

// ---- fast path for rows of 8K+ keys: a sampled threshold and one pass over HBM -------------
// A histogram of every kSampleStride-th 128-byte line of the row places a value bin b_est below
// the k-th largest score with a margin of a few standard deviations; one pass then gathers every
// element of bin >= b_est into the LDS list (slots reserved with one LDS atomic per wave and
// load group, so the list is in no particular order).  The exact threshold bin is found on the
// list and its elements ranked pairwise by (key desc, index asc); the kept positions are marked
// in an LDS bitmap and written in index order.  Any miss (too few or too many candidates, a
// crowded threshold bin) returns false before anything is written, and the exact two-pass path
// runs instead, so the result never depends on the sample.
constexpr int kSampleStride = 8;                          // sample one 128-byte line in 8
// A score below every element of value bin >= b (value_bin is monotone, so any x with
// value_bin(x) < b will do): lo + (b - 0.01)/sc, moved down by ulps until value_bin confirms it.
// The pass then tests x > floor with one compare per element, gathering bins >= b and at most
// a sliver of bin b-1 (the finish rejects the list unless its threshold bin is >= b).
__device__ __forceinline__ float bin_floor_below(int b, float lo, float sc) {
  if (b <= 0) return -__builtin_inff();
  float x = lo + (float(b) - 0.01f) / sc;
  for (int it = 0; it < 64; ++it) {
    if (value_bin(x, lo, sc, kVBins) < b) return x;
    x = key_to_score(score_key(x) - 1u);  // next float down
  }
  return -__builtin_inff();  // every element a candidate: the list overflows, the exact path runs
}

constexpr int kFastMinN = 8192;                           // shorter rows: the exact path
constexpr int kFastMaxN = int(sizeof(decltype(TopkRowSmem::u))) * 8;  // bitmap bits in the union

// Sampled threshold bin of a row whose scores lie in [lo, lo + kVBins/sc].  The sample is every
// kSampleStride-th whole 128-byte line of the row (counted from the first 128-byte boundary in
// it), so no sampled line drags in bytes that are not used.  The bin leaves z standard
// deviations of the sampled count (plus 4) as margin above k.  Returns 0 (every element a
// candidate) when the sample is too small to place the margin.  BATCH line loads per thread are
// issued before their histogram atomics.  Every thread of the block must call it; all get the
// same result.
template <int BATCH>
__device__ __forceinline__ int sample_threshold(const float* __restrict__ row, int n, int K, float lo, float sc,
                                                float z, TopkSmem& s) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kVBins; i += kTopkThreads) s.hist[i] = 0;
  __syncthreads();
  const int skip = int(((128u - (uint32_t(reinterpret_cast<uintptr_t>(row)) & 127u)) & 127u) >> 2);
  const int nlines = n > skip ? (n - skip) >> 5 : 0;  // whole 32-float lines after the boundary
  const int nsl = (nlines + kSampleStride - 1) / kSampleStride;
  const float* base = row + skip;
  for (int m0 = 0; m0 < nsl; m0 += BATCH * kTopkThreads) {
    f32x4 x[BATCH][8];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int m = m0 + u * kTopkThreads + tid;
      if (m < nsl) {
        const float* p = base + (int64_t)m * kSampleStride * 32;
#pragma unroll
        for (int c = 0; c < 8; ++c) x[u][c] = *reinterpret_cast<const f32x4*>(p + 4 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
      if (m0 + u * kTopkThreads + tid < nsl)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) atomicAdd(&s.hist[value_bin(x[u][c][e], lo, sc, kVBins)], 1);
  }
  __syncthreads();
  const int ns = 32 * nsl;
  const float expect = float(K) * float(ns) / float(n);
  const int need = int(expect + z * sqrtf(expect) + 4.f);
  if (need > ns) return 0;
  find_digit(s, kVBins, need);
  return s.sel_digit;
}

// keys/ids (LDS) hold `total` (K <= total <= CAP) candidates of a row of n <= kFastMaxN scores,
// in any order, among them every element whose value bin is >= b_est (and possibly some of
// lower bins).  Finds the exact threshold bin b1, ranks its elements, and writes the k selected
// positions in index order; b1 < b_est (the list's bins >= b_est hold fewer than k) fails.  `bits` (kFastMaxN / 32 words of LDS) may alias keys/ids: the kept positions are moved
// to registers first.  Each kept position then finds its output slot directly: the exclusive
// count of 4-word bitmap groups before it (a block scan, stored in s.hist) plus at most four
// popcounts -- balanced however the selection clusters.  Returns false, with nothing written,
// when bin b1 is too crowded to rank in LDS.
static_assert(kFastMaxN / 128 <= kBins, "bitmap group counts must fit the histogram array");

template <int CAP, class BinOf>
__device__ __forceinline__ bool finish_unordered(int n, int K, BinOf bin_of, int b_est, int total,
                                                 uint32_t* keys, int* ids, uint32_t* bits, int32_t* __restrict__ out,
                                                 TopkSmem& s, FinishSmem<512>& f) {
  static_assert(CAP % kTopkThreads == 0, "list capacity must be a multiple of the block size");
  const int tid = threadIdx.x;
  for (int i = tid; i < kVBins; i += kTopkThreads) s.hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < total; i += kTopkThreads) atomicAdd(&s.hist[bin_of(keys[i])], 1);
  __syncthreads();
  find_digit(s, kVBins, K);
  const int b1 = s.sel_digit, above = s.sel_above;
  if (b1 < b_est) return false;  // bins below b_est may be incomplete in the list
  if (!rank_threshold_bin(keys, ids, total, b1, K - above, bin_of, f)) return false;
  // kept = bin > b1, or bin == b1 and not rejected (rejected keys were set to 0)
  constexpr int PER = CAP / kTopkThreads;
  int kept[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int i = tid + kTopkThreads * c;
    kept[c] = -1;
    if (i < total) {
      const uint32_t k = keys[i];
      if (k != 0u && bin_of(k) >= b1) kept[c] = ids[i];
    }
  }
  __syncthreads();
  const int nwords = (n + 31) >> 5;
  for (int i = tid; i < nwords; i += kTopkThreads) bits[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < PER; ++c)
    if (kept[c] >= 0) atomicOr(&bits[kept[c] >> 5], 1u << (kept[c] & 31));
  __syncthreads();
  // exclusive counts of 4-word groups: thread t scans groups [t*gpt, t*gpt + gpt)
  const int ngroups = (nwords + 3) >> 2;
  const int gpt = (ngroups + kTopkThreads - 1) / kTopkThreads;
  const int g0 = min(ngroups, tid * gpt), g1 = min(ngroups, g0 + gpt);
  auto group_count = [&](int g) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * g + q < nwords) c += __popc(bits[4 * g + q]);
    return c;
  };
  int cnt = 0;
  for (int g = g0; g < g1; ++g) cnt += group_count(g);
  int tot;
  const int incl = block_incl_scan(cnt, s.wave_tot, &tot);
  int run = incl - cnt;
  for (int g = g0; g < g1; ++g) {
    s.hist[g] = run;  // the histogram is no longer needed; ngroups <= kBins
    run += group_count(g);
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int id = kept[c];
    if (id >= 0) {
      const int w = id >> 5, g = w >> 2;
      int pos = s.hist[g] + __popc(bits[w] & ((1u << (id & 31)) - 1u));
      for (int q = 4 * g; q < w; ++q) pos += __popc(bits[q]);
      out[pos] = id;
    }
  }
  return true;
}

__device__ bool select_row_fast(const float* __restrict__ row, int n, int K, float lo, float sc,
                                int32_t* __restrict__ out, TopkRowSmem& sm) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  if (tid == 0) sm.s.list_n = 0;
  const int b_est = sample_threshold<1>(row, n, K, lo, sc, 3.f, sm.s);
  const float floor_est = bin_floor_below(b_est, lo, sc);
  // one pass: every element above floor_est (all of bin >= b_est) into the list
  const int seg = (((n + kTopkWaves - 1) / kTopkWaves) + 3) & ~3;
  const int seg_lo = min(n, w * seg), seg_hi = min(n, seg_lo + seg);
  constexpr int STEPW = 256 * kQ;
  for (int base = seg_lo; base < seg_hi; base += STEPW) {
    f32x4 v[kQ];
    load_step(row, base, seg_hi, lane, v, -__builtin_inff());
#pragma unroll
    for (int e = 0; e < kQ; ++e) {
      const int i0 = base + 4 * (lane + 64 * e);
      bool keep[4];
      int before = 0, total = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        keep[j] = v[e][j] > floor_est;  // slots past the segment hold -inf
        const uint64_t bm = __ballot(keep[j]);
        before += lanes_below(bm);
        total += __popcll(bm);
      }
      if (total == 0) continue;
      int bpos = 0;
      if (lane == 0) bpos = atomicAdd(&sm.s.list_n, total);
      int slot = __shfl(bpos, 0) + before;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (keep[j]) {
          if (slot < kListCap) {
            sm.u.l.lkeys[slot] = score_key(v[e][j]);
            sm.u.l.lids[slot] = i0 + j;
          }
          ++slot;
        }
    }
  }
  __syncthreads();
  const int total = sm.s.list_n;
  if (total < K || total > kListCap) return false;
  auto bin_of = [&](uint32_t k) { return value_bin(key_to_score(k), lo, sc, kVBins); };
  return finish_unordered<kListCap>(n, K, bin_of, b_est, total, sm.u.l.lkeys, sm.u.l.lids,
                                    reinterpret_cast<uint32_t*>(&sm.u), out, sm.s, sm.f);
}

// Exact select of a row with n > K and hi > lo: two passes over the row (per-wave value
// histograms, then an ordered compaction of the threshold bin and above), with radix passes over
// HBM for rows whose candidates overflow the LDS list.
__device__ __forceinline__ void select_row_exact(const float* __restrict__ row, int n, int K, float lo, float hi,
                                 int32_t* __restrict__ out, TopkRowSmem& sm) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const float sc = float(kVBins) / (hi - lo);
  // wave w owns the contiguous segment [seg_lo, seg_hi) (starts are multiples of 4 elements)
  const int seg = (((n + kTopkWaves - 1) / kTopkWaves) + 3) & ~3;
  const int seg_lo = min(n, w * seg), seg_hi = min(n, seg_lo + seg);
  constexpr int STEPW = 256 * kQ;  // elements per wave step

  // pass 1: per-wave histograms of the value bins
  for (int i = tid; i < kTopkWaves * kVBins; i += kTopkThreads) (&sm.u.whist[0][0])[i] = 0;
  if (tid < kTopkWaves) sm.wcnt[tid] = 0;
  __syncthreads();
  for (int base = seg_lo; base < seg_hi; base += STEPW) {
    f32x4 v[kQ];
    load_step(row, base, seg_hi, lane, v);
#pragma unroll
    for (int e = 0; e < kQ; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (base + 4 * (lane + 64 * e) + j < seg_hi) atomicAdd(&sm.u.whist[w][value_bin(v[e][j], lo, sc, kVBins)], 1);
  }
  __syncthreads();
  for (int b = tid; b < kVBins; b += kTopkThreads) {
    int a = 0;
#pragma unroll
    for (int ww = 0; ww < kTopkWaves; ++ww) a += sm.u.whist[ww][b];
    sm.s.hist[b] = a;
  }
  __syncthreads();
  find_digit(sm.s, kVBins, K);
  const int b1 = sm.s.sel_digit;
  // candidates per wave: elements whose bin >= b1
  {
    int c[kTopkWaves];
#pragma unroll
    for (int ww = 0; ww < kTopkWaves; ++ww) c[ww] = 0;
    for (int b = b1 + tid; b < kVBins; b += kTopkThreads)
#pragma unroll
      for (int ww = 0; ww < kTopkWaves; ++ww) c[ww] += sm.u.whist[ww][b];
#pragma unroll
    for (int ww = 0; ww < kTopkWaves; ++ww) c[ww] = wave_sum_i(c[ww]);
    if (lane == 0)
#pragma unroll
      for (int ww = 0; ww < kTopkWaves; ++ww) atomicAdd(&sm.wcnt[ww], c[ww]);
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int ww = 0; ww < kTopkWaves; ++ww) {
        sm.woff[ww] = acc;
        acc += sm.wcnt[ww];
      }
      sm.s.list_n = acc;
    }
    __syncthreads();
  }
  const int cand = sm.s.list_n;
  uint32_t prefix = 0, hmask = 0;
  int krem = K;
  if (cand <= kListCap) {
    // pass 2: each wave compacts its segment's candidates, in index order, at its offset
    int pos = sm.woff[w];
    for (int base = seg_lo; base < seg_hi; base += STEPW) {
      f32x4 v[kQ];
      load_step(row, base, seg_hi, lane, v);
#pragma unroll
      for (int e = 0; e < kQ; ++e) {
        const int i0 = base + 4 * (lane + 64 * e);
        bool keep[4];
        int before = 0, total = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          keep[j] = (i0 + j < seg_hi) && value_bin(v[e][j], lo, sc, kVBins) >= b1;
          const uint64_t bm = __ballot(keep[j]);
          before += lanes_below(bm);
          total += __popcll(bm);
        }
        int slot = pos + before;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (keep[j]) {
            sm.u.l.lkeys[slot] = score_key(v[e][j]);
            sm.u.l.lids[slot] = i0 + j;
            ++slot;
          }
        pos += total;
      }
    }
    __syncthreads();
    const int above = sm.s.sel_above;
    auto bin_of = [&](uint32_t k) { return value_bin(key_to_score(k), lo, sc, kVBins); };
    if (rank_threshold_bin(sm.u.l.lkeys, sm.u.l.lids, cand, b1, K - above, bin_of, sm.f)) {
      emit_nonzero(sm.u.l.lkeys, sm.u.l.lids, cand, out, sm.s);
    } else {
      const ListSrc ls{sm.u.l.lkeys, sm.u.l.lids};
      radix_rest(ls, cand, 0, prefix, hmask, krem, sm.s);
      ordered_emit(ls, cand, prefix, krem, [&](int slot, uint32_t, int id) { out[slot] = id; }, sm.s);
    }
  } else {
    const RowSrc src{row, true};
    radix_rest(src, n, 0, prefix, hmask, krem, sm.s);
    ordered_emit(src, n, prefix, krem, [&](int slot, uint32_t, int id) { out[slot] = id; }, sm.s);
  }
}

__device__ void select_row(const float* __restrict__ row, int n, int K, float lo, float hi,
                           int32_t* __restrict__ out, TopkRowSmem& sm) {
  if (n <= K || !(hi > lo)) {  // everything kept, or every score equal: the first k keys win
    first_k(n, K, out);
    return;
  }
  if (n >= kFastMinN && n <= kFastMaxN && select_row_fast(row, n, K, lo, float(kVBins) / (hi - lo), out, sm))
    return;
  __syncthreads();  // the fast path's LDS is reused below
  select_row_exact(row, n, K, lo, hi, out, sm);
}

// Prefill rows of one chunk of 16-row blocks: slot c of the chunk buffer holds the block at
// position n0 + c of the chunked loop (schedule entry chunk_entry(n0 + c), rows with a stride of
// 16(j+1) floats); one workgroup per (slot, row), in slot order.
__global__ __launch_bounds__(kTopkThreads) void topk_prefill_kernel(
    const float* __restrict__ buf, int64_t slot_stride, const int2* __restrict__ sched,
    const int* __restrict__ sched_count, int n0, const int32_t* __restrict__ cu, int K,
    const float2* __restrict__ rowrange, int32_t* __restrict__ out) {
  __shared__ TopkRowSmem sm;
  const int slot = blockIdx.x >> 4, rr = blockIdx.x & 15;
  const int n = n0 + slot;
  const int N = *sched_count;
  if (n >= N) return;
  const int2 e = sched[chunk_entry(n, N)];
  const int b = e.x, j = e.y, i = 16 * j + rr;
  if (i >= cu[b + 1] - cu[b]) return;
  const int64_t t = cu[b] + i;
  const float* row = buf + (int64_t)slot * slot_stride + (int64_t)rr * 16 * (j + 1);
  const float2 rg = rowrange[t];
  select_row(row, i + 1, K, rg.x, rg.y, out + t * K, sm);
}

// ------------------------------------------------------------------------------------------
// Standalone top-k over general float32 rows (the deterministic stand-in for torch.topk).
// NaN (any payload) and -inf are masked: key 0.  Every other value keeps its order-preserving
// key, which is >= 0x00800000 (the key of -FLT_MAX), so the top 11-bit digit of a selectable
// key is >= 4 and digit 0 counts masked elements only.
// One workgroup per row, each wave owning a contiguous quarter of it:
//   pass 1   per-wave histograms of the top digit -> #selectable, threshold digit d1;
//   pass 1b  only when digit d1 would leave too many candidates for LDS: per-wave histograms of
//            the second digit among elements whose top digit is d1 (threshold now 22 bits);
//   pass 2   ordered compaction of every key >= the threshold prefix into an LDS list;
//   finish   radix select of the remaining digits on the list, ordered emit to the output.
// Rows with more candidates than the list holds even after pass 1b (massive ties) run the
// remaining digits and the emit over HBM.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t general_key(float x) {
  return (x != x || x == -__builtin_inff()) ? 0u : score_key(x);
}

struct GenRowSrc {
  const float* __restrict__ row;
  bool vec;  // 16-byte aligned
  __device__ __forceinline__ void quad(int n, int s0, uint32_t* keys, int* ids) const {
    if (vec && s0 + 3 < n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + s0);
#pragma unroll
      for (int e = 0; e < 4; ++e) keys[e] = general_key(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) keys[e] = (s0 + e < n) ? general_key(row[s0 + e]) : 0u;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ids[e] = s0 + e;
  }
};

constexpr int kGenListCap = 4096;

struct TopkGenSmem {
  TopkSmem s;
  union {
    int whist[kTopkWaves][kBins];  // per-wave digit histograms
    struct {
      uint32_t lkeys[kGenListCap];  // candidate list (index order)
      int lids[kGenListCap];
    } l;
  } u;
  int wcnt[kTopkWaves];
  int woff[kTopkWaves];
};

// One wave step of kQ float4 per lane over [base, base + 256 kQ); slots at or past hi are 0.
template <bool VEC>
__device__ __forceinline__ void gen_load_step(const float* __restrict__ row, int base, int hi, int lane,
                                              f32x4 (&v)[kQ]) {
#pragma unroll
  for (int e = 0; e < kQ; ++e) {
    const int i = base + 4 * (lane + 64 * e);
    if (VEC && i + 3 < hi) {
      v[e] = *reinterpret_cast<const f32x4*>(row + i);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[e][j] = (i + j < hi) ? row[i + j] : 0.f;
    }
  }
}

// Per-wave histogram over [lo, hi): bin = dig(key), skipped when negative.
template <bool VEC, class Dig>
__device__ __forceinline__ void gen_wave_hist(const float* __restrict__ row, int lo, int hi, int lane, int* wh,
                                              Dig dig) {
  for (int base = lo; base < hi; base += 256 * kQ) {
    f32x4 v[kQ];
    gen_load_step<VEC>(row, base, hi, lane, v);
#pragma unroll
    for (int e = 0; e < kQ; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (base + 4 * (lane + 64 * e) + j < hi) {
          const int d = dig(general_key(v[e][j]));
          if (d >= 0) atomicAdd(&wh[d], 1);
        }
  }
}

// Per-wave ordered compaction over [lo, hi) of the elements with keep(key): put(slot, key, id)
// with slots counting up from pos in index order.
template <bool VEC, class Keep, class Put>
__device__ __forceinline__ void gen_wave_compact(const float* __restrict__ row, int lo, int hi, int lane, int pos,
                                                 Keep keep_fn, Put put) {
  for (int base = lo; base < hi; base += 256 * kQ) {
    f32x4 v[kQ];
    gen_load_step<VEC>(row, base, hi, lane, v);
#pragma unroll
    for (int e = 0; e < kQ; ++e) {
      const int i0 = base + 4 * (lane + 64 * e);
      bool keep[4];
      uint32_t key[4];
      int before = 0, total = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        key[j] = general_key(v[e][j]);
        keep[j] = (i0 + j < hi) && keep_fn(key[j]);
        const uint64_t bm = __ballot(keep[j]);
        before += lanes_below(bm);
        total += __popcll(bm);
      }
      int slot = pos + before;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (keep[j]) put(slot++, key[j], i0 + j);
      pos += total;
    }
  }
}

// Sum the per-wave histograms into sm.s.hist.
__device__ __forceinline__ void gen_merge_hist(TopkGenSmem& sm) {
  for (int b = threadIdx.x; b < kBins; b += kTopkThreads) {
    int a = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) a += sm.u.whist[w][b];
    sm.s.hist[b] = a;
  }
  __syncthreads();
}

// Per-wave counts of the bins [from, kBins) into sm.wcnt (added), then exclusive offsets in
// sm.woff and the total in sm.s.list_n.
__device__ __forceinline__ void gen_wave_counts(TopkGenSmem& sm, int from, bool add) {
  const int lane = threadIdx.x & 63;
  int c[kTopkWaves];
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) c[w] = 0;
  for (int b = from + threadIdx.x; b < kBins; b += kTopkThreads)
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) c[w] += sm.u.whist[w][b];
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) c[w] = wave_sum_i(c[w]);
  if (!add && threadIdx.x < kTopkWaves) sm.wcnt[threadIdx.x] = 0;
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) atomicAdd(&sm.wcnt[w], c[w]);
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      sm.woff[w] = acc;
      acc += sm.wcnt[w];
    }
    sm.s.list_n = acc;
  }
  __syncthreads();
}

// ---- fast path of the standalone top-k: a sampled key threshold and one pass over HBM -------
// As the prefill fast path, but with no score range known: the sample (every kSampleStride-th
// 128-byte line) is binned on the order-preserving key, top 11 bits and then the next 11 bits
// inside the chosen digit, giving a threshold key T with a margin of three standard deviations
// of the sampled count.  One pass gathers every element with key >= T (a float compare against
// the score whose key is T: NaN and -inf never pass) into the unordered LDS list, which
// finish_unordered settles exactly with key bins (k - T) >> sh.  Any miss returns false before
// anything is written and the two-pass path runs.
constexpr int kGenFastMaxK = 2048;  // the list (kListCap) must hold k plus the margin

template <class Dig>
__device__ __forceinline__ void gen_sample_hist(const float* __restrict__ base, int nsl, Dig dig, TopkSmem& s) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kBins; i += kTopkThreads) s.hist[i] = 0;
  __syncthreads();
  for (int m = tid; m < nsl; m += kTopkThreads) {
    const float* p = base + (int64_t)m * kSampleStride * 32;
    f32x4 x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = *reinterpret_cast<const f32x4*>(p + 4 * c);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = dig(general_key(x[c][e]));
        if (d >= 0) atomicAdd(&s.hist[d], 1);
      }
  }
  __syncthreads();
}

__device__ bool select_general_fast(const float* __restrict__ row, int n, int K, int32_t* __restrict__ out,
                                    TopkRowSmem& sm) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int skip = int(((128u - (uint32_t(reinterpret_cast<uintptr_t>(row)) & 127u)) & 127u) >> 2);
  const int nlines = n > skip ? (n - skip) >> 5 : 0;
  const int nsl = (nlines + kSampleStride - 1) / kSampleStride;
  const int ns = 32 * nsl;
  const float expect = float(K) * float(ns) / float(n);
  const int need = int(expect + 3.f * sqrtf(expect) + 4.f);
  if (need > ns) return false;
  const float* base = row + skip;
  gen_sample_hist(base, nsl, [](uint32_t k) { return int(k >> 21); }, sm.s);
  find_digit(sm.s, kBins, need);
  const int d1 = sm.s.sel_digit, above1 = sm.s.sel_above;
  gen_sample_hist(base, nsl, [d1](uint32_t k) { return int(k >> 21) == d1 ? int((k >> 10) & 0x7FFu) : -1; }, sm.s);
  find_digit(sm.s, kBins, need - above1);
  const uint32_t T = (uint32_t(d1) << 21) | (uint32_t(sm.s.sel_digit) << 10);
  if (T <= 0x007FFFFFu) return false;  // at or below the key of -inf: masked elements would pass
  const float xT = key_to_score(T);    // the score whose key is T (NaN when T is a NaN key: nothing passes)
  if (tid == 0) sm.s.list_n = 0;
  __syncthreads();
  const int seg = (((n + kTopkWaves - 1) / kTopkWaves) + 3) & ~3;
  const int seg_lo = min(n, w * seg), seg_hi = min(n, seg_lo + seg);
  constexpr int STEPW = 256 * kQ;
  for (int b0 = seg_lo; b0 < seg_hi; b0 += STEPW) {
    f32x4 v[kQ];
    load_step(row, b0, seg_hi, lane, v, -__builtin_inff());
#pragma unroll
    for (int e = 0; e < kQ; ++e) {
      const int i0 = b0 + 4 * (lane + 64 * e);
      bool keep[4];
      int before = 0, total = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        keep[j] = v[e][j] >= xT;  // slots past the segment hold -inf, which never passes
        const uint64_t bm = __ballot(keep[j]);
        before += lanes_below(bm);
        total += __popcll(bm);
      }
      if (total == 0) continue;
      int bpos = 0;
      if (lane == 0) bpos = atomicAdd(&sm.s.list_n, total);
      int slot = __shfl(bpos, 0) + before;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (keep[j]) {
          if (slot < kListCap) {
            sm.u.l.lkeys[slot] = score_key(v[e][j]);
            sm.u.l.lids[slot] = i0 + j;
          }
          ++slot;
        }
    }
  }
  __syncthreads();
  const int total = sm.s.list_n;
  if (total < K || total > kListCap) return false;
  // key bins relative to T, fine enough that the largest key lands in bin < kVBins
  uint32_t kmax = 0u;
  for (int i = tid; i < total; i += kTopkThreads) kmax = max(kmax, sm.u.l.lkeys[i]);
  for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  if (lane == 0) sm.s.wave_tot[w] = int(kmax - T);
  __syncthreads();
  uint32_t span = 0u;
#pragma unroll
  for (int ww = 0; ww < kTopkWaves; ++ww) span = max(span, uint32_t(sm.s.wave_tot[ww]));
  __syncthreads();
  int sh = 0;
  while ((span >> sh) >= uint32_t(kVBins)) ++sh;
  auto bin_of = [T, sh](uint32_t k) { return min(kVBins - 1, int((k - T) >> sh)); };
  return finish_unordered<kListCap>(n, K, bin_of, 0, total, sm.u.l.lkeys, sm.u.l.lids,
                                    reinterpret_cast<uint32_t*>(&sm.u), out, sm.s, sm.f);
}

template <bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_general_kernel(const float* __restrict__ scores, int64_t ld,
                                                                    int n_all, const int32_t* __restrict__ lens,
                                                                    int K, int32_t* __restrict__ out) {
  __shared__ union {
    TopkGenSmem g;  // two-pass path
    TopkRowSmem f;  // sampled single pass
  } smu;
  TopkGenSmem& sm = smu.g;
  const int64_t r = blockIdx.x;
  const float* __restrict__ row = scores + r * ld;
  const int n = lens ? max(0, min(n_all, lens[r])) : n_all;
  int32_t* __restrict__ orow = out + r * K;
  if constexpr (VEC) {
    if (n >= kFastMinN && n <= kFastMaxN && K <= kGenFastMaxK && select_general_fast(row, n, K, orow, smu.f))
      return;  // exactly k positions written
    __syncthreads();  // the fast path's LDS is reused below
  }
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int seg = (((n + kTopkWaves - 1) / kTopkWaves) + 3) & ~3;
  const int seg_lo = min(n, w * seg), seg_hi = min(n, seg_lo + seg);

  // pass 1: top digit
  for (int i = tid; i < kTopkWaves * kBins; i += kTopkThreads) (&sm.u.whist[0][0])[i] = 0;
  __syncthreads();
  gen_wave_hist<VEC>(row, seg_lo, seg_hi, lane, sm.u.whist[w], [](uint32_t k) { return int(k >> 21); });
  __syncthreads();
  gen_merge_hist(sm);
  const int nvalid = n - sm.s.hist[0];
  const int kp = min(K, nvalid);
  if (kp == nvalid) {
    // every selectable element is kept: compact them straight into the output
    gen_wave_counts(sm, 1, false);
    gen_wave_compact<VEC>(row, seg_lo, seg_hi, lane, sm.woff[w], [](uint32_t k) { return k != 0u; },
                          [&](int slot, uint32_t, int id) { orow[slot] = id; });
  } else {
    find_digit(sm.s, kBins, kp);
    const int d1 = sm.s.sel_digit;
    int krem = kp - sm.s.sel_above;
    uint32_t prefix = uint32_t(d1) << 21, hmask = 0x7FFu << 21;
    int d0 = 1;
    gen_wave_counts(sm, d1, false);  // candidates per wave: top digit >= d1
    if (sm.s.list_n > kGenListCap) {
      // pass 1b: refine inside digit d1 with the second digit
      gen_wave_counts(sm, d1 + 1, false);  // keep only the surely-kept part (top digit > d1)
      for (int i = tid; i < kTopkWaves * kBins; i += kTopkThreads) (&sm.u.whist[0][0])[i] = 0;
      __syncthreads();
      gen_wave_hist<VEC>(row, seg_lo, seg_hi, lane, sm.u.whist[w],
                         [d1](uint32_t k) { return int(k >> 21) == d1 ? int((k >> 10) & 0x7FFu) : -1; });
      __syncthreads();
      gen_merge_hist(sm);
      find_digit(sm.s, kBins, krem);
      const int d2 = sm.s.sel_digit;
      krem -= sm.s.sel_above;
      prefix |= uint32_t(d2) << 10;
      hmask |= 0x7FFu << 10;
      d0 = 2;
      gen_wave_counts(sm, d2, true);  // + elements of digit d1 whose second digit >= d2
    }
    const int cand = sm.s.list_n;
    if (cand <= kGenListCap) {
      // pass 2: every key >= prefix (higher bits above the threshold, or equal so far)
      gen_wave_compact<VEC>(row, seg_lo, seg_hi, lane, sm.woff[w], [prefix](uint32_t k) { return k >= prefix; },
                            [&](int slot, uint32_t key, int id) {
                              sm.u.l.lkeys[slot] = key;
                              sm.u.l.lids[slot] = id;
                            });
      __syncthreads();
      const ListSrc ls{sm.u.l.lkeys, sm.u.l.lids};
      radix_rest(ls, cand, d0, prefix, hmask, krem, sm.s);
      ordered_emit(ls, cand, prefix, krem, [&](int slot, uint32_t, int id) { orow[slot] = id; }, sm.s);
    } else {
      const GenRowSrc src{row, VEC};
      radix_rest(src, n, d0, prefix, hmask, krem, sm.s);
      ordered_emit(src, n, prefix, krem, [&](int slot, uint32_t, int id) { orow[slot] = id; }, sm.s);
    }
  }
  for (int s2 = kp + tid; s2 < K; s2 += kTopkThreads) orow[s2] = -1;
}

hipError_t launch_topk_general(const float* scores, int64_t rows, int n, int64_t ld, const int32_t* lens, int K,
                               int32_t* out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const bool vec = (reinterpret_cast<uintptr_t>(scores) & 15) == 0 && ld % 4 == 0;
  if (vec)
    topk_general_kernel<true><<<(unsigned)rows, kTopkThreads, 0, st>>>(scores, ld, n, lens, K, out);
  else
    topk_general_kernel<false><<<(unsigned)rows, kTopkThreads, 0, st>>>(scores, ld, n, lens, K, out);
  return hipGetLastError();
}

hipError_t launch_topk_prefill(const float* buf, int64_t slot_stride, const int2* sched, const int* count, int n0,
                               int nblocks, const int32_t* cu, int K, const float2* rowrange, int32_t* out,
                               hipStream_t st) {
  if (nblocks <= 0) return hipSuccess;
  topk_prefill_kernel<<<(unsigned)nblocks * 16, kTopkThreads, 0, st>>>(buf, slot_stride, sched, count, n0, cu, K,
                                                                      rowrange, out);
  return hipGetLastError();
}

}  // namespace dsa
