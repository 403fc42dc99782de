// Decode top-k selection: one 1024-thread workgroup per sequence picks the first min(k, n) of its n
// cached keys in the order (score descending, index ascending) and writes them in ascending index
// order, -1 padded (Keye-VL-2.0 summary page, gsyq.cn, section 一: keep the 2048 most relevant
// positions; section 八: a deterministic selection).
//
// Scores map to order-preserving uint32 keys; bin(key) = key >> kDecodeBinShift (16 bins per
// octave of the score).  The decode indexer leaves, per block of kDecodeKeysPerBlock keys, its keys
// sorted by bin (highest first, the keys below its window last) with their positions, and a
// histogram window of kDecodeWinBins bins from its base (the octave of its largest key and the
// three below) holding, per bin, how many of its keys lie in that bin or above.  With B* the
// highest base of the row, every block counts every key of bin >= B*, so the summed windows give
// exact counts of keys at or above each bin >= B*.  When B* itself has at least k keys at or above
// it, the threshold bin T1 (holding the k-th largest key) is the highest bin that does, and every
// key of bin >= T1 is at the head of its block's sorted list (the block's window count at T1 says
// how many): the workgroup copies exactly those heads into an LDS list
// (about k plus one bin), each thread a few entries.  A radix select over the low bits of T1's
// entries gives the exact k-th key T and how many keys equal to T are kept (lowest positions
// first).  The output slot of a kept entry is its rank in position order: bitmaps of the kept
// positions (keys > T, keys == T) with per-word prefix counts give it with one popcount, so the
// entries are written in parallel.  Rows where the windows do not reach k keys, or whose list
// would overflow, run the same radix select and emit over all the blocks' lists (exact, slower).
// Integer LDS atomics only; the result does not depend on timing.
#include "common.h"

namespace dsa {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelCap = 8192;                          // LDS candidate list entries
constexpr int kSelMaxBlocks = 4096;                    // indexer blocks per row (2^20 keys)
// histogram windows staged in LDS per round: 640 x 128 bytes fill the union with the emit
// bitmaps, so a row of up to 163840 keys (a 128K context plus its generated tokens) sums its
// windows in one round (at 512, a 131136-key row paid a second round for its 513th window)
constexpr int kStageWins = 640;
constexpr int kEmitPos = 5 * 32 * 1024;                 // positions per emit round (5 words per thread)
constexpr int kEmitWords = kEmitPos / 32;
constexpr int kEmitWordsPerThread = kEmitWords / kSelThreads;
constexpr int kBlocksPerThread = kSelMaxBlocks / kSelThreads;
static_assert(kEmitWordsPerThread * kSelThreads == kEmitWords, "whole bitmap words per thread");
static_assert(kBlocksPerThread * kSelThreads == kSelMaxBlocks, "whole blocks per thread");
static_assert(kDecodeKeysPerBlock == 256, "block positions are 8 bits");

struct SelSmem {
  union {
    struct {
      uint32_t key[kSelCap];
      int pos[kSelCap];
    } list;
    int bases[kSelMaxBlocks];  // histogram window bases, until the list is filled
  } a;
  union {
    uint16_t stage[kStageWins * kDecodeWinBins];  // windows of one round
    int cpre[kSelMaxBlocks + 1];                  // list offset of each block's candidates
    struct {
      uint32_t gt[kEmitWords], eq[kEmitWords];    // kept positions: keys > T, keys == T
      int pgt[kEmitWords], peq[kEmitWords];       // exclusive prefix counts per word
    } e;
  } b;
  int hist[2048];
  int wtot[kSelWaves];
  int wtot2[kSelWaves];
  int digit, above, t1, t1_above;
};

// Block-wide inclusive scan over the 1024 threads; *total = block sum.
__device__ __forceinline__ int sel_scan(int v, int* wtot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wtot[wave] = incl;
  lds_sync();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = wtot[w];
    before += (w < wave) ? t : 0;
    tot += t;
  }
  lds_sync();
  *total = tot;
  return incl + before;
}

// ---- element sources: the LDS candidate list, or every block's sorted list in global memory ----
struct SelList {
  const uint32_t* keys;
  const int* pos;
  __device__ __forceinline__ void quad(int m, int s0, uint32_t (&k)[4], int (&p)[4]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = s0 + e < m;
      k[e] = ok ? keys[s0 + e] : 0u;
      p[e] = ok ? pos[s0 + e] : -1;
    }
  }
};

// Entry i of a row's block lists: block i / 256, slot i % 256; the block holds min(256, n - 256 *
// block) keys.  Lists are 16-byte aligned (keys) and 4-byte aligned (positions) per block.
struct SelBlocks {
  const uint32_t* __restrict__ keys;
  const uint8_t* __restrict__ pos;
  int n;
  __device__ __forceinline__ void quad(int m, int s0, uint32_t (&k)[4], int (&p)[4]) const {
    const int s = s0 < m ? s0 : 0;
    const i32x4 kv = *reinterpret_cast<const i32x4*>(keys + s);
    const uint32_t pv = *reinterpret_cast<const uint32_t*>(pos + s);
    const int blk = s0 >> 8, valid = min(kDecodeKeysPerBlock, n - (blk << 8));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = s0 + e < m && ((s0 + e) & 255) < valid;
      k[e] = ok ? uint32_t(kv[e]) : 0u;
      p[e] = ok ? (blk << 8) + int((pv >> (8 * e)) & 255u) : -1;
    }
  }
};

// One radix digit: among elements with (key & hmask) == prefix, the digit (key >> shift) & (2^width
// - 1) holding the krem-th largest key.  Updates prefix, hmask and krem (krem becomes the rank
// still to take inside the chosen digit).  Elements with p < 0 are absent.
template <class Src>
__device__ void sel_digit(const Src& src, int m, uint32_t& prefix, uint32_t& hmask, int& krem, int shift, int width,
                          SelSmem& sm) {
  const int nb = 1 << width, tid = threadIdx.x;
  const uint32_t dmask = uint32_t(nb - 1);
  for (int i = tid; i < nb; i += kSelThreads) sm.hist[i] = 0;
  lds_sync();
  for (int c0 = 0; c0 < m; c0 += 4 * kSelThreads) {
    uint32_t k[4];
    int p[4];
    src.quad(m, c0 + 4 * tid, k, p);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (p[e] >= 0 && (k[e] & hmask) == prefix) atomicAdd(&sm.hist[(k[e] >> shift) & dmask], 1);
  }
  lds_sync();
  // digits in descending order: thread t takes bins [top - bpt, top), top = nb - bpt * t
  const int bpt = nb > kSelThreads ? nb / kSelThreads : 1;
  const int top = nb - bpt * tid;
  int local = 0;
  for (int i = 1; i <= bpt; ++i)
    if (top - i >= 0) local += sm.hist[top - i];
  int total;
  const int incl = sel_scan(local, sm.wtot, &total);
  const int excl = incl - local;
  if (excl < krem && krem <= incl) {
    int c = excl;
    for (int i = 1; i <= bpt; ++i) {
      const int h = sm.hist[top - i];
      if (c + h >= krem) {
        sm.digit = top - i;
        sm.above = c;
        break;
      }
      c += h;
    }
  }
  lds_sync();
  krem -= sm.above;
  prefix |= uint32_t(sm.digit) << shift;
  hmask |= dmask << shift;
  lds_sync();
}

// Writes, in ascending position order, every element with key > T and the krem lowest-position
// elements with key == T.  Positions lie in [0, n).  visit(w0, w1, f) calls f(key, pos) for the
// source elements with positions in [w0, w1), each position at most once; it is called twice per
// round of kEmitPos positions (marking, then writing).
template <class Visit>
__device__ void sel_emit(int n, uint32_t T, int krem, Visit visit, int32_t* __restrict__ orow, SelSmem& sm) {
  const int tid = threadIdx.x;
  int base_gt = 0, base_eq = 0;
  for (int w0 = 0; w0 < n; w0 += kEmitPos) {
    const int w1 = min(n, w0 + kEmitPos);
#pragma unroll
    for (int j = 0; j < kEmitWordsPerThread; ++j) {
      sm.b.e.gt[tid * kEmitWordsPerThread + j] = 0u;
      sm.b.e.eq[tid * kEmitWordsPerThread + j] = 0u;
    }
    lds_sync();
    visit(w0, w1, [&](uint32_t k, int p) {
      const int q = p - w0;
      if (k > T) atomicOr(&sm.b.e.gt[q >> 5], 1u << (q & 31));
      else if (k == T) atomicOr(&sm.b.e.eq[q >> 5], 1u << (q & 31));
    });
    lds_sync();
    int cg[kEmitWordsPerThread], ce[kEmitWordsPerThread], sg = 0, se = 0;
#pragma unroll
    for (int j = 0; j < kEmitWordsPerThread; ++j) {
      cg[j] = __popc(sm.b.e.gt[tid * kEmitWordsPerThread + j]);
      ce[j] = __popc(sm.b.e.eq[tid * kEmitWordsPerThread + j]);
      sg += cg[j];
      se += ce[j];
    }
    int tg, te;
    int xg = base_gt + sel_scan(sg, sm.wtot, &tg) - sg;
    int xe = base_eq + sel_scan(se, sm.wtot2, &te) - se;
#pragma unroll
    for (int j = 0; j < kEmitWordsPerThread; ++j) {
      sm.b.e.pgt[tid * kEmitWordsPerThread + j] = xg;
      sm.b.e.peq[tid * kEmitWordsPerThread + j] = xe;
      xg += cg[j];
      xe += ce[j];
    }
    lds_sync();
    visit(w0, w1, [&](uint32_t k, int p) {
      if (k < T) return;
      const int q = p - w0, wd = q >> 5;
      const uint32_t below = (1u << (q & 31)) - 1u;
      const int rg = sm.b.e.pgt[wd] + __popc(sm.b.e.gt[wd] & below);  // kept keys > T before p
      const int re = sm.b.e.peq[wd] + __popc(sm.b.e.eq[wd] & below);  // keys == T before p
      if (k > T) orow[rg + min(re, krem)] = p;
      else if (re < krem) orow[rg + re] = p;
    });
    base_gt += tg;
    base_eq += te;
    lds_sync();
  }
}

}  // namespace

__global__ __launch_bounds__(kSelThreads) void topk_decode_select_kernel(
    const uint32_t* __restrict__ skeys, const uint8_t* __restrict__ spos, const int32_t* __restrict__ cache_lens,
    int max_len, int K, const int* __restrict__ wbase, const uint16_t* __restrict__ wcnt, int blk_stride,
    int32_t* __restrict__ out) {
  __shared__ SelSmem sm;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = min(max(0, cache_lens[b]), max_len);  // lengths past max_len break the caller's contract
  int32_t* __restrict__ orow = out + (int64_t)b * K;
  if (n <= K) {
    for (int s = tid; s < K; s += kSelThreads) orow[s] = (s < n) ? s : -1;
    return;
  }
  const int nblk = (n + kDecodeKeysPerBlock - 1) / kDecodeKeysPerBlock;
  const int64_t row0 = (int64_t)b * blk_stride;
  const int* __restrict__ wb = wbase + row0;
  const uint16_t* __restrict__ wc = wcnt + row0 * kDecodeWinBins;
  const uint32_t* __restrict__ kb = skeys + row0 * kDecodeKeysPerBlock;
  const uint8_t* __restrict__ pb = spos + row0 * kDecodeKeysPerBlock;
  constexpr int kPieces = kDecodeWinBins * 2 / 16;                  // 16-byte pieces per window
  constexpr int kStageLoads = kStageWins * kPieces / kSelThreads;   // per thread and round

  // ---- window bases (and the first round of windows, requested together) -------------------
  i32x4 v[kStageLoads];
  const int cnt0 = min(kStageWins, nblk);
#pragma unroll
  for (int i = 0; i < kStageLoads; ++i) {
    const int pc = tid + kSelThreads * i;
    if (pc / kPieces < cnt0) v[i] = *reinterpret_cast<const i32x4*>(wc + pc * 8);
  }
  int bmax = -(1 << 30);
#pragma unroll
  for (int i = 0; i < kBlocksPerThread; ++i) {
    const int w = tid + kSelThreads * i;
    if (w < nblk) {
      const int bw = wb[w];
      sm.a.bases[w] = bw;
      bmax = max(bmax, bw);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) bmax = max(bmax, __shfl_xor(bmax, o));
  if (lane == 0) sm.wtot[wave] = bmax;
  if (tid < kDecodeWinBins) sm.hist[tid] = 0;
  lds_sync();
  int bstar = sm.wtot[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) bstar = max(bstar, sm.wtot[w]);

  // ---- exact counts of keys at or above bins B* .. B* + kDecodeWinBins - 1 ----------------
  for (int w0 = 0; w0 < nblk; w0 += kStageWins) {
    const int cnt = min(kStageWins, nblk - w0);
    if (w0 > 0) {
#pragma unroll
      for (int i = 0; i < kStageLoads; ++i) {
        const int pc = tid + kSelThreads * i;
        if (pc / kPieces < cnt) v[i] = *reinterpret_cast<const i32x4*>(wc + (w0 * kPieces + pc) * 8);
      }
    }
    lds_sync();  // the previous round's sums have read the staging area
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) {
      const int pc = tid + kSelThreads * i;
      if (pc / kPieces < cnt) *reinterpret_cast<i32x4*>(sm.b.stage + pc * 8) = v[i];
    }
    lds_sync();
    const int j = tid % kDecodeWinBins, grp = tid / kDecodeWinBins;
    constexpr int kGroups = kSelThreads / kDecodeWinBins;
    int acc = 0;
#pragma unroll 8
    for (int wi = grp; wi < cnt; wi += kGroups) {
      const int idx = j + bstar - sm.a.bases[w0 + wi];  // >= 0: B* >= every base
      acc += idx < kDecodeWinBins ? int(sm.b.stage[wi * kDecodeWinBins + idx]) : 0;
    }
    if (acc) atomicAdd(&sm.hist[j], acc);
  }
  lds_sync();

  // ---- threshold bin T1: the highest bin with at least k keys at or above it ---------------
  static_assert(kDecodeWinBins == 64, "one wave lane per window bin");
  if (wave == 0) {
    const int c = sm.hist[lane];
    const uint64_t reach = __ballot(c >= K);
    if (lane == 0) sm.t1 = -1;
    if (reach) {
      const int jt = 63 - __builtin_clzll(reach);
      const int above = __shfl(c, min(jt + 1, 63));
      if (lane == 0) {
        sm.t1 = bstar + jt;
        sm.t1_above = jt < 63 ? above : 0;
      }
    }
  }
  lds_sync();
  const int t1 = sm.t1;

  if (t1 >= 0) {
    // ---- candidates per block: its keys of bin >= T1 (the head of its sorted list) ---------
    // (windows of the last round are still staged in LDS; earlier ones are read again)
    const int last0 = (nblk - 1) / kStageWins * kStageWins;
    int cw[kBlocksPerThread], ctot = 0;
#pragma unroll
    for (int i = 0; i < kBlocksPerThread; ++i) {
      const int w = kBlocksPerThread * tid + i;  // contiguous blocks per thread: prefix in block order
      int c = 0;
      if (w < nblk) {
        const int j0 = t1 - sm.a.bases[w];       // >= 0: T1 >= B* >= every base
        if (j0 < kDecodeWinBins)
          c = w >= last0 ? int(sm.b.stage[(w - last0) * kDecodeWinBins + j0]) : int(wc[(int64_t)w * kDecodeWinBins + j0]);
      }
      cw[i] = c;
      ctot += c;
    }
    int m;
    int x = sel_scan(ctot, sm.wtot, &m) - ctot;
    if (m <= kSelCap) {
#pragma unroll
      for (int i = 0; i < kBlocksPerThread; ++i) {
        const int w = kBlocksPerThread * tid + i;
        if (w < nblk) sm.b.cpre[w] = x;
        x += cw[i];
      }
      if (tid == 0) sm.b.cpre[nblk] = m;
      lds_sync();
      // copy list entries, several per thread with their loads issued together; entry e belongs
      // to the last block w with cpre[w] <= e (a fixed-step bisection written as selects)
      constexpr int PER = kSelCap / kSelThreads;
      for (int e0 = 0; e0 < m; e0 += PER * kSelThreads) {
        int blk[PER], src[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          const int e = min(e0 + u * kSelThreads + tid, m - 1);
          int lo = 0;
#pragma unroll
          for (int step = kSelMaxBlocks / 2; step > 0; step >>= 1) {
            const int c = min(lo + step, nblk);
            lo = (sm.b.cpre[c] <= e) ? c : lo;
          }
          blk[u] = lo;
          src[u] = lo * kDecodeKeysPerBlock + (e - sm.b.cpre[lo]);
        }
        uint32_t kv[PER];
        uint32_t pv[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          kv[u] = kb[src[u]];
          pv[u] = pb[src[u]];
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          const int e = e0 + u * kSelThreads + tid;
          if (e < m) {
            sm.a.list.key[e] = kv[u];
            sm.a.list.pos[e] = blk[u] * kDecodeKeysPerBlock + int(pv[u]);
          }
        }
      }
      lds_sync();
      // ---- exact threshold inside bin T1, then the ordered emit from the list ---------------
      uint32_t prefix = uint32_t(t1) << kDecodeBinShift, hmask = ~((1u << kDecodeBinShift) - 1u);
      int krem = K - sm.t1_above;
      const SelList ls{sm.a.list.key, sm.a.list.pos};
      sel_digit(ls, m, prefix, hmask, krem, 8, kDecodeBinShift - 8, sm);
      // the entries sharing the top 24 key bits of the k-th key: usually a handful of exact ties.
      // Rank them directly by (key descending, position ascending); the dropped ones get key 0
      // and every kept entry then has a key > prefix - 1, which the emit keeps whole.
      const int gn = sm.hist[sm.digit];
      if (gn <= kSelThreads) {
        int* gidx = sm.b.cpre;  // free again: the list is complete
        if (tid == 0) sm.above = 0;
        lds_sync();
        for (int i = tid; i < m; i += kSelThreads)
          if ((sm.a.list.key[i] & hmask) == prefix) gidx[atomicAdd(&sm.above, 1)] = i;
        lds_sync();
        int drop = -1;
        if (tid < gn) {
          const int i = gidx[tid];
          const uint32_t k = sm.a.list.key[i];
          const int p = sm.a.list.pos[i];
          int rank = 0;
          for (int x = 0; x < gn; ++x) {
            const int ix = gidx[x];
            const uint32_t kx = sm.a.list.key[ix];
            rank += (kx > k) | ((kx == k) & (sm.a.list.pos[ix] < p));
          }
          if (rank >= krem) drop = i;
        }
        lds_sync();
        if (drop >= 0) sm.a.list.key[drop] = 0u;
        lds_sync();
        prefix -= 1u;
        krem = 0;
      } else {
        sel_digit(ls, m, prefix, hmask, krem, 0, 8, sm);
      }
      sel_emit(n, prefix, krem, [&](int w0, int w1, auto f) {
        for (int i = tid; i < m; i += kSelThreads) {
          const int p = sm.a.list.pos[i];
          if (p >= w0 && p < w1) f(sm.a.list.key[i], p);
        }
      }, orow, sm);
      return;
    }
  }

  // ---- exact select over every block's list (windows short of k keys, or the list overflowed) --
  const SelBlocks bs{kb, pb, n};
  const int total = nblk * kDecodeKeysPerBlock;
  uint32_t prefix = 0, hmask = 0;
  int krem = K;
  sel_digit(bs, total, prefix, hmask, krem, 21, 11, sm);
  sel_digit(bs, total, prefix, hmask, krem, 10, 11, sm);
  sel_digit(bs, total, prefix, hmask, krem, 0, 10, sm);
  sel_emit(n, prefix, krem, [&](int w0, int w1, auto f) {
    // every entry of the blocks that hold positions [w0, w1)
    const int e1 = min(total, (w1 + kDecodeKeysPerBlock - 1) / kDecodeKeysPerBlock * kDecodeKeysPerBlock);
    for (int c0 = w0; c0 < e1; c0 += 4 * kSelThreads) {
      uint32_t k[4];
      int p[4];
      bs.quad(e1, c0 + 4 * tid, k, p);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (p[e] >= 0) f(k[e], p[e]);
    }
  }, orow, sm);
}

// The decode indexer's block lists and windows of row b start at block b * blk_stride.
hipError_t launch_topk_decode(const uint32_t* skeys, const uint8_t* spos, const int32_t* cache_lens, int B,
                              int max_len, int K, const int* wbase, const uint16_t* wcnt, int blk_stride,
                              int32_t* out, hipStream_t st) {
  if ((reinterpret_cast<uintptr_t>(skeys) & 15) != 0 || (reinterpret_cast<uintptr_t>(wcnt) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(spos) & 3) != 0)
    return hipErrorInvalidValue;
  if (blk_stride < (max_len + kDecodeKeysPerBlock - 1) / kDecodeKeysPerBlock || blk_stride > kSelMaxBlocks)
    return hipErrorInvalidValue;
  topk_decode_select_kernel<<<B, kSelThreads, 0, st>>>(skeys, spos, cache_lens, max_len, K, wbase, wcnt,
                                                       blk_stride, out);
  return hipGetLastError();
}

}  // namespace dsa
