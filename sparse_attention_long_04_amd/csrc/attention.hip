// Sparse GQA attention over the selected keys, and the dense causal reference
// (Keye-VL-2.0 summary page, gsyq.cn, section 一: attention only among the selected positions;
// the base LLM uses GQA; costs are quoted against standard full attention).
//
// attend_staged (the per-wave body shared by both gather kernels) -- one wave attends one row
//   for one KV head; the head's query heads (Hq/Hkv, padded to 16) share the row's index set.
//   Per 32-key tile:
//     S^T = K Q^T   bf16 MFMA 16x16x32, K rows gathered from HBM into the wave's LDS (direct
//                     loads, 64 contiguous bytes per quad) and read back as A operands;
//     online softmax in fp32 (exp2, running max/sum per head);
//     O^T += V^T P^T  bf16 MFMA 16x16x32 with P split as hi + lo bf16 (two MFMAs, relative
//                     error ~2^-16).  V needs keys along the MFMA k dimension: each lane
//                     gathers 8 keys x 8 consecutive dims and the head-dim order is permuted
//                     (dim tile dt holds dims 8*row + dt), so the transpose happens inside the
//                     lane's registers -- no LDS round trip for V.
//   The next tile's K/V rows are loaded while the current one is computed; the row's key
//   indices are staged in LDS first.
//
// gather_rows_kernel (prefill) -- XCD- and cache-aware: the launch runs the KV heads one after
//   another (phases in launch order); within a phase workgroup b runs on XCD b % 8 and its 4
//   waves take 4 consecutive rows, chunks of consecutive row groups dealt round-robin over the
//   XCDs.  Each XCD's L2 then holds one head's K/V rows (512 B per key instead of 2 KiB) of
//   neighbouring rows, and all XCDs work on the same stretch of rows of the same head, whose K/V
//   rows (67 MB at 128K) fit the memory-side Infinity Cache that they share.
//
// gather_attention_kernel (decode, dense decode, and prefill shapes the row kernel does not
//   take) -- one workgroup per row and key split, one wave per KV head.  With several splits
//   the wave writes (unnormalised O, running max, sum) partials that combine_kernel merges by
//   log-sum-exp; with one split it writes bf16 output directly.  idx == nullptr means
//   "keys 0..n-1" (dense decode).
//
// dense_prefill_kernel -- FlashAttention-style causal attention: a workgroup of 8 waves owns
//   128 query tokens x 2 query heads of one KV group; 64-key K and V^T tiles are copied straight
//   into LDS rings and shared by both heads; S^T and O^T use 32x32x16 MFMAs (bf16 for QK, fp16
//   for PV from a V^T copy in fp16 made once per call), software-pipelined over half tiles.
#include "attn_tiles.h"

namespace dsa {

struct RowInfo {
  int64_t kv_row0;  // row of key 0 in the K/V arrays (units of Hkv*D elements)
  int n;            // causal context length
};

__device__ __forceinline__ RowInfo row_info(int mode, int64_t r, const int32_t* cu, int nseq,
                                            const int32_t* cache_lens, int cap) {
  RowInfo ri;
  if (mode == 0) {
    const int b = find_seq(cu, nseq, r);
    ri.kv_row0 = cu[b];
    ri.n = int(r - cu[b]) + 1;
  } else {
    ri.kv_row0 = r * (int64_t)cap;
    ri.n = cache_lens[r];
  }
  return ri;
}

constexpr int kMaxSplitKeys = 4096;  // LDS index slots per workgroup

// bf16 pair (lo from a, hi from b): element e of 8-element vectors a and b.
__device__ __forceinline__ uint32_t pair_bf16(const i32x4& a, const i32x4& b, int e) {
  const uint32_t x = uint32_t(a[e >> 1]), y = uint32_t(b[e >> 1]);
  return (e & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
}

// K tile of the LDS path: load (h, c) of the wave lands in region 4h+c, each lane's 16 bytes at
// lane*16; the 16-byte pad per region staggers the banks of the transposed read-back.
constexpr int kKRegion = 64 * 16 + 16;
constexpr int kKTileLds = 8 * kKRegion;  // per wave

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm8 = 0x0F78;     // vmcnt(8), others not waited
constexpr int kWaitLgkm0 = 0xC07F;   // lgkmcnt(0), others not waited

template <int D, bool LAZY>
__device__ __forceinline__ void attend_staged(const uint16_t* __restrict__ q, const int* __restrict__ il, int cnt32,
                                              int64_t r, int g, int G, int Hq, int64_t kvs,
                                              const uint16_t* __restrict__ kg_base,
                                              const uint16_t* __restrict__ vg_base, float scale_log2, int lr, int lg,
                                              f32x4 (&o)[8], float& m_run, float& l_tot,
                                              __attribute__((address_space(3))) uint8_t* kb) {
  i32x4 qf[4];
  {
    const bool hv = lr < G;
    const uint16_t* qp = q + (r * Hq + g * G + (hv ? lr : 0)) * D + 32 * lg;  // dims 32lg + 8c, as K
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qf[c] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(qp + 8 * c));
      if (!hv) qf[c] = (i32x4){0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  m_run = -__builtin_inff();
  float l_run = 0.f;

  // One tile of 32 keys.  Lane (lr, lg):
  //   kf[h][c]: K row of key slot 8(lr/4)+4h+(lr%4), dims 32lg+8c .. +7  (S^T A operand; the
  //             contraction runs over the dims in this order, and Q is loaded the same way)
  //   vf[m]   : V row of key slot 8lg+m, dims 8lr .. 8lr+7             (transposed in registers)
  //   sv[m]   : index of key slot 8lg+m (-1 = masked)
  auto compute = [&](const i32x4 (&kf)[2][4], const i32x4 (&vf)[8], const int (&sv)[8]) {
    // ---- S^T = K Q^T for the two 16-key sub-tiles; lane slot 8lg + 4h + i
    float z[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) c4 = mfma_bf16_16x16x32(kf[h][c], qf[c], c4);
#pragma unroll
      for (int i = 0; i < 4; ++i) z[4 * h + i] = (sv[4 * h + i] >= 0) ? c4[i] * scale_log2 : -__builtin_inff();
    }
    // ---- online softmax (per head = lane column; keys over registers and the 4 lane groups).
    // LAZY: the reference max moves only when a head's tile max passes it by more than 8 (log2
    // units), so p = 2^(z - m) <= 2^8 and the O rescale -- a round trip of the accumulators
    // through VALU -- happens on few tiles (it costs registers: the decode kernel keeps the
    // eager form to stay at two waves per SIMD).
    float mt = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, z[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if constexpr (LAZY) {
      const bool move = mt > m_run + 8.f;  // false while every key so far is masked
      if (__ballot(move)) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;  // m_run = -inf: 0
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
        m_run = move ? mt : m_run;
      }
    } else {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - ((m_new == -__builtin_inff()) ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;
    float ps = 0.f;
    uint32_t phi[8], plo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = __builtin_amdgcn_exp2f(z[i] - m_use);
      ps += pv;
      // p = hi + lo: hi = p truncated to bf16, lo = the remainder truncated to bf16
      const uint32_t hb = __float_as_uint(pv) & 0xFFFF0000u;
      phi[i] = hb;
      plo[i] = __float_as_uint(pv - __uint_as_float(hb)) & 0xFFFF0000u;
    }
    l_run += ps;
    const i32x4 bh = {int((phi[0] >> 16) | phi[1]), int((phi[2] >> 16) | phi[3]), int((phi[4] >> 16) | phi[5]),
                      int((phi[6] >> 16) | phi[7])};
    const i32x4 bl = {int((plo[0] >> 16) | plo[1]), int((plo[2] >> 16) | plo[3]), int((plo[4] >> 16) | plo[5]),
                      int((plo[6] >> 16) | plo[7])};
    // ---- O^T += V^T P^T; dim tile dt holds dims 8*row + dt, row = 0..15
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const i32x4 a = {int(pair_bf16(vf[0], vf[1], dt)), int(pair_bf16(vf[2], vf[3], dt)),
                       int(pair_bf16(vf[4], vf[5], dt)), int(pair_bf16(vf[6], vf[7], dt))};
      o[dt] = mfma_bf16_16x16x32(a, bh, o[dt]);
      o[dt] = mfma_bf16_16x16x32(a, bl, o[dt]);
    }
  };

  {
    // K through LDS.  In the MFMA layout above the four lanes of a quad hold four different
    // keys, so loading K straight into it would make every 16-byte load touch four rows per
    // quad (the address unit pays per row).  Instead the tile's 8 K loads go straight to the
    // wave's LDS regions (load (h, c): lane (4a+i, lg) fetches key slot 8a+4h+c, dims
    // 32lg+8i -- 64 contiguous bytes per quad) and are read back in the MFMA layout (lane
    // (4a+i, lg), register c of sub-tile h = region (h, i), lane slot 4a+c+16lg), with no VALU
    // transpose.  Per tile the K loads are issued before the V loads: at the top of the next
    // iteration vmcnt(8) leaves only the V loads in flight.  A region is refilled only after
    // its read-back has completed (lgkmcnt(0)).
    struct VTile {
      i32x4 vf[8];
      int sv[8];
    };
    // Gather addresses: the head's K/V base is wave-uniform and a key's byte offset from it,
    // index * row bytes, fits 32 bits (the launchers check the sequence / cache length), so each
    // load takes a scalar base plus one 24-bit multiply-add per lane.
    const uint32_t rowb = uint32_t(kvs) * 2;
    const char* const kgb = reinterpret_cast<const char*>(kg_base);
    const char* const vgb = reinterpret_cast<const char*>(vg_base);
    const uint32_t klane = 2 * (32 * lg + 8 * (lr & 3)), vlane = 16 * lr;
    auto issue = [&](VTile& t, int tl) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const i32x4 sk = *reinterpret_cast<const i32x4*>(il + tl + 8 * (lr >> 2) + 4 * h);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          __builtin_amdgcn_global_load_lds(kgb + (__umul24(uint32_t(max(sk[c], 0)), rowb) + klane),
                                           kb + (4 * h + c) * kKRegion, 16, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the K loads ahead of the V loads (vmcnt order)
      const i32x4 s0 = *reinterpret_cast<const i32x4*>(il + tl + 8 * lg);
      const i32x4 s1 = *reinterpret_cast<const i32x4*>(il + tl + 8 * lg + 4);
#pragma unroll
      for (int m = 0; m < 4; ++m) { t.sv[m] = s0[m]; t.sv[4 + m] = s1[m]; }
#pragma unroll
      for (int m = 0; m < 8; ++m)
        t.vf[m] = *reinterpret_cast<const i32x4*>(vgb + (__umul24(uint32_t(max(t.sv[m], 0)), rowb) + vlane));
    };
    const __attribute__((address_space(3))) uint8_t* kr = kb + (lr & 3) * kKRegion + (4 * (lr >> 2) + 16 * lg) * 16;
    // tile tl: its V rows are in `cur` (loaded during the previous tile), the next tile's go to
    // `nxt`; the loop alternates the two register sets instead of copying one into the other
    auto step = [&](int tl, const VTile& cur, VTile& nxt) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitVm8);  // this tile's K is in LDS
      i32x4 kf[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          kf[h][c] = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(kr + 4 * h * kKRegion + 16 * c);
      if (tl + 32 < cnt32) {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the read-back has landed
        __builtin_amdgcn_sched_barrier(0);
        issue(nxt, tl + 32);
      }
      compute(kf, cur.vf, cur.sv);
    };
    VTile va, vb;
    if (cnt32 > 0) issue(va, 0);
    for (int tl = 0; tl < cnt32; tl += 64) {
      step(tl, va, vb);
      if (tl + 32 < cnt32) step(tl + 32, vb, va);
    }
  }
  l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
}

// Normalised bf16 output of head `head` (lane column) from the attend_staged accumulators.
template <int D>
__device__ __forceinline__ void store_out_bf16(uint16_t* __restrict__ out, int64_t r, int Hq, int head, int lg,
                                               const f32x4 (&o)[8], float l_tot) {
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  uint16_t* op = out + (r * Hq + head) * D + 32 * lg;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    i32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = int(uint32_t(f32_to_bf16(o[2 * e][i] * inv)) | (uint32_t(f32_to_bf16(o[2 * e + 1][i] * inv)) << 16));
    __builtin_nontemporal_store(w, reinterpret_cast<i32x4*>(op + 8 * i));
  }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, (8 + NW - 1) / NW) void gather_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, int K, int mode, const int32_t* __restrict__ cu, int nseq,
    const int32_t* __restrict__ cache_lens, int cap, int Hq, int Hkv, float scale_log2,
    int keys_per_split, int nsplit, uint16_t* __restrict__ out, float* __restrict__ o_part,
    float2* __restrict__ ml_part, float* __restrict__ lse_out) {
  static_assert(D == 128, "head_dim 128 only");
  __shared__ __attribute__((aligned(16))) int il[kMaxSplitKeys + 32];
  __shared__ __attribute__((aligned(16))) uint8_t kb_all[NW][kKTileLds];  // K tiles (LDS path)
  const int64_t r = blockIdx.x;
  const int split = blockIdx.y;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int G = Hq / Hkv;
  const RowInfo ri = row_info(mode, r, cu, nseq, cache_lens, cap);
  const int m_all = idx ? min(K, ri.n) : ri.n;
  const int p_begin = split * keys_per_split;
  const int p_end = min(m_all, p_begin + keys_per_split);
  const int cnt = max(0, p_end - p_begin);
  const int cnt32 = (cnt + 31) & ~31;

  // stage this split's key indices in LDS; slots past the end hold -1
  for (int j = threadIdx.x; j < cnt32; j += 64 * NW) {
    int s = -1;
    if (j < cnt) s = idx ? __builtin_nontemporal_load(idx + r * K + p_begin + j) : p_begin + j;
    il[j] = s;
  }
  __syncthreads();

  const int64_t kvs = (int64_t)Hkv * D;
  f32x4 o[8];
  float m_run, l_tot;
  attend_staged<D, false>(q, il, cnt32, r, g, G, Hq, kvs, k + ri.kv_row0 * kvs + g * D,
                                v + ri.kv_row0 * kvs + g * D, scale_log2, lr, lg, o, m_run, l_tot,
                                (__attribute__((address_space(3))) uint8_t*)kb_all[g]);
  if (lr >= G) return;
  const int head = g * G + lr;
  if (nsplit == 1) {
    store_out_bf16<D>(out, r, Hq, head, lg, o, l_tot);
    if (lse_out && lg == 0) lse_out[r * Hq + head] = (m_run + __log2f(l_tot)) * 0.6931471805599453f;
  } else {
    const int64_t slot = (r * nsplit + split) * Hq + head;
    float* pp = o_part + slot * D + 32 * lg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 a = {o[0][i], o[1][i], o[2][i], o[3][i]};
      f32x4 b = {o[4][i], o[5][i], o[6][i], o[7][i]};
      *reinterpret_cast<f32x4*>(pp + 8 * i) = a;
      *reinterpret_cast<f32x4*>(pp + 8 * i + 4) = b;
    }
    if (lg == 0) ml_part[slot] = make_float2(m_run, l_tot);
  }
}

// Prefill variant with an XCD-aware mapping.  The grid is Hkv / hp phases of blocks_per_phase
// workgroups (a multiple of 8); phase p serves heads p*hp .. p*hp + hp - 1 over all rows.  Within
// a phase, workgroup b runs on XCD b % 8 (the dispatcher deals workgroups round-robin over the 8
// XCDs), serves head p*hp + (b % 8) % hp, and its NW waves take NW consecutive rows, each staging
// its own indices; chunks of kGatherChunk consecutive row groups go to consecutive XCDs.  Every XCD gathers the K/V
// rows of a single head (Hkv * 256 B less per key than a workgroup spanning all heads), and the
// heads in flight at once are only hp.  `order` (optional) maps slots to rows: rows whose
// selections share a key block are then gathered together.  Needs 8 % Hkv == 0 and K <= kRowKeys.
constexpr int kRowKeys = 2048;
// KV heads gathered at once.  One head at a time (in head order) keeps the working set of K/V
// rows to one head's (67 MB at 128K tokens): measured at 128K, 4 heads at once 59.8 ms, 2 heads
// 56.0, 1 head 55.4.
constexpr int kGatherHeadsPerPhase = 1;
// Row groups per chunk dealt to one XCD: consecutive rows on one XCD keep the keys that
// neighbouring rows share in its L2.  Measured in natural row order (attention ms, 128K
// i.i.d. / drifting queries): 1 group 55.8 / 46.1, 4: 55.8 / 41.6, 16: 55.4 / 39.8, 32: 55.4 /
// 39.7, 64: 55.3 / 39.7; with the rows in dominant-block order (i.i.d.): 16: 41.6, 32: 41.5,
// 64: 41.2, 128: 41.1, 256: 41.1, 512: 41.2.
constexpr int kGatherChunk = 128;

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, (8 + NW - 1) / NW) void gather_rows_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, int K, const int32_t* __restrict__ cu, int nseq, int64_t rows, int Hq,
    int Hkv, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse_out, int hp,
    unsigned blocks_per_phase, const int32_t* __restrict__ order) {
  static_assert(D == 128, "head_dim 128 only");
  __shared__ __attribute__((aligned(16))) int il_all[NW][kRowKeys + 32];
  __shared__ __attribute__((aligned(16))) uint8_t kb_all[NW][kKTileLds];  // K tiles (LDS path)
  // phase p (in launch order) serves heads p*hp .. p*hp+hp-1 over all rows
  const unsigned phase = blockIdx.x / blocks_per_phase, bid = blockIdx.x % blocks_per_phase;
  const int xcd = bid & 7;  // blocks_per_phase is a multiple of 8: the XCD of the workgroup
  const int g = int(phase) * hp + xcd % hp;
  // row groups are dealt to the 8 / hp XCDs of a head in chunks of kGatherChunk consecutive groups
  const int64_t slot = bid >> 3;
  const int64_t group = (slot / kGatherChunk) * (8 / hp) * kGatherChunk + (xcd / hp) * kGatherChunk + slot % kGatherChunk;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rslot = group * NW + wave;
  if (rslot >= rows) return;  // waves are independent: no workgroup barrier below
  // the row this slot serves (wave-uniform)
  const int64_t r = order ? (int64_t)__builtin_amdgcn_readfirstlane(order[rslot]) : rslot;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int G = Hq / Hkv;
  const RowInfo ri = row_info(0, r, cu, nseq, nullptr, 0);
  const int cnt = min(K, ri.n);
  const int cnt32 = (cnt + 31) & ~31;
  int* il = il_all[wave];
  for (int j = lane; j < cnt32; j += 64) il[j] = (j < cnt) ? __builtin_nontemporal_load(idx + r * K + j) : -1;
  __builtin_amdgcn_wave_barrier();  // the wave's own LDS writes precede its reads (in-order LDS)

  const int64_t kvs = (int64_t)Hkv * D;
  f32x4 o[8];
  float m_run, l_tot;
  attend_staged<D, true>(q, il, cnt32, r, g, G, Hq, kvs, k + ri.kv_row0 * kvs + g * D,
                               v + ri.kv_row0 * kvs + g * D, scale_log2, lr, lg, o, m_run, l_tot,
                               (__attribute__((address_space(3))) uint8_t*)kb_all[wave]);
  if (lr >= G) return;
  store_out_bf16<D>(out, r, Hq, g * G + lr, lg, o, l_tot);
  // natural-log log-sum-exp of the row's scaled scores (the backward's softmax statistics)
  if (lse_out && lg == 0) lse_out[r * Hq + g * G + lr] = (m_run + __log2f(l_tot)) * 0.6931471805599453f;
}

// Merge split partials: out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).  Splits are read
// in batches of kCombineBatch whose loads are all issued before any is used, with a running
// maximum carried across batches; empty splits (l_s == 0) contribute nothing.
constexpr int kCombineBatch = 16;

__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ o_part,
                                                      const float2* __restrict__ ml_part, int nsplit, int Hq,
                                                      int D, uint16_t* __restrict__ out) {
  const int64_t r = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x;
  float M = -__builtin_inff(), L = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += kCombineBatch) {
    float m[kCombineBatch], l[kCombineBatch], o[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int s = s0 + u;
      m[u] = -__builtin_inff();
      l[u] = 0.f;
      o[u] = 0.f;
      if (s < nsplit) {
        const int64_t slot = (r * nsplit + s) * Hq + h;
        const float2 ml = ml_part[slot];
        m[u] = ml.x;
        l[u] = ml.y;
        o[u] = o_part[slot * D + d];
      }
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      if (l[u] != 0.f) Mb = fmaxf(Mb, m[u]);
    if (Mb == -__builtin_inff()) continue;  // nothing non-empty so far
    const float rescale = exp2f(M - Mb);    // 0 while M is still -inf
    L *= rescale;
    acc *= rescale;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (l[u] != 0.f) {
        const float wgt = exp2f(m[u] - Mb);
        L += l[u] * wgt;
        acc += o[u] * wgt;
      }
    }
    M = Mb;
  }
  out[(r * Hq + h) * D + d] = f32_to_bf16(L > 0.f ? acc / L : 0.f);
}

// ------------------------------------------------------------------------------------------
// Dense causal prefill (FlashAttention-style), head_dim 128.
// Workgroup = 128 query tokens x HW query heads of one KV group (HW = 2 when the group size is
// even, else 1), 4 HW waves: wave w takes tokens 32(w%4) .. +31 of head w/4.
//
// K and V^T tiles of 64 keys are copied from global memory straight into LDS (one 16-byte unit
// per lane and copy instruction), each in a ring of three stages; Q stays in registers.  V is
// read from a fp16 V^T copy (dims x keys) made once per call, so the A operand of
// O^T += V^T P^T comes from plain 16-byte LDS reads (transposing LDS reads move under half the
// bytes per cycle).  A K row (one key) is 256 bytes with its 16-byte unit u at unit
// u ^ dn_swz(row); a V^T row (one dim) is 128 bytes with unit u at u ^ ((row / 2) % 8).  Both
// layouts keep every operand read free of LDS bank conflicts (16 lanes fetch the same unit of
// 16 consecutive rows, which land on 16 distinct bank groups).
//
// Software pipeline over 32-key half tiles.  Iteration t runs two half steps; each issues 8 QK
// MFMAs of the next half (S), 8 PV MFMAs of the previous half (O^T += V^T P^T) and the 16
// exponentials of the current half (P = 2^(S scale - m), fp16, with per-lane row sums),
// interleaved one MFMA and one exponential per step behind scheduling barriers, so the matrix
// cores always have work that does not wait for the vector ALUs and the exponentials spread
// over every MFMA:
//   half step A: S(t, keys 32..63) | P(t, keys 0..31)  | O += V(t-1, 32..63) P(t-1, 32..63)
//   half step B: S(t+1, keys 0..31) | P(t, keys 32..63) | O += V(t, 0..31) P(t, 0..31)
// The reference m is lazy: it is set from tile 0's row maxima and moves only when some lane's
// sum of P over a half tile exceeds 2^15 (which keeps every P inside fp16's range); that half's
// scores are then recomputed from K(t), still in its stage, O (holding the halves before it) and
// the row sums rescaled to the new maxima and its P redone.
// ------------------------------------------------------------------------------------------
constexpr int kDnTileB = 64 * 256;    // one 64-key tile of K or V^T
constexpr int kDnKst = 0;             // K stages at 0, 16K, 32K
constexpr int kDnVst = 3 * kDnTileB;  // V^T stages at 48K, 64K, 80K
constexpr int kDnLds = 6 * kDnTileB;  // 96 KB

__device__ __forceinline__ int dn_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// First column of sequence b (first token cub) in the V^T rows: round64(cu[b]) + 128 b -- 64-column
// aligned, so 8-key units are 16-byte aligned, and at least 64 columns past the previous
// sequence's last token; those 64 columns are zeros, so a key tile that runs past a sequence's
// end reads zeros, never another sequence's values.
__device__ __host__ __forceinline__ int64_t dn_vt_base(int64_t cub, int b) {
  return (cub + 63) / 64 * 64 + 128 * int64_t(b);
}

template <int HW>
__global__ __launch_bounds__(256 * HW) void dense_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ vt, int64_t tpad,
    const int32_t* __restrict__ cu, int Hq, int Hkv, float scale_log2, const int2* __restrict__ sched,
    const int* __restrict__ sched_count, uint16_t* __restrict__ out) {
  constexpr int D = 128, BM = 128, BN = 64, NW = 4 * HW;
  constexpr int CPW = 16 / NW;  // 1 KB copies per wave and tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kDnLds];
  const int n = blockIdx.x;
  if (n >= *sched_count) return;
  const int2 e = sched[n];
  const int b = e.x, j = e.y;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = HW * blockIdx.y + (w >> 2);  // the wave's head (the workgroup's heads share a KV head)
  const int g = h / G;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int q0 = BM * j;
  const int kend = min(q0 + BM, L);     // keys 0 .. kend-1: the block's last query is kend-1
  const int nt = (kend + BN - 1) / BN;  // key tiles of the workgroup
  const int qc = lane & 31, hf = lane >> 5;
  const int64_t kvs = (int64_t)Hkv * D;
  const int wq0 = q0 + 32 * (w & 3);                        // the wave's first query
  const int my_q = min(wq0 + qc, kend - 1);                 // lanes past the end repeat the last
  const int wlast = (wq0 < kend) ? (wq0 + 31) / BN : -1;    // the wave's last tile
  lds_u8* const lb = (lds_u8*)lds;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lb;

  // Q (B operand of S^T = K Q^T) in registers: lane (qc, hf) holds dims 16 s2 + 8 hf .. +7
  i32x4 qf[8];
  {
    const uint16_t* qp = q + ((seq0 + my_q) * Hq + h) * D + 8 * hf;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) qf[s2] = *reinterpret_cast<const i32x4*>(qp + 16 * s2);
  }

  // K tile copy: this wave fills rows 4 CPW w + 4x + lane/16 (x < CPW) of a stage, one unit per
  // lane (keys past the block's end repeat its last key; their scores are masked).  Byte offsets
  // from the sequence's first row fit 32 bits (the launcher checks the K/V size).
  const int dr = 4 * CPW * w + (lane >> 4);
  const uint32_t rowb = uint32_t(kvs) * 2;
  const uint16_t* const kg = k + seq0 * kvs + g * D;
  auto copy_k = [&](int stage, int tile) {
    const uint32_t dst = lds0 + kDnKst + stage * kDnTileB + 1024 * CPW * w;
#pragma unroll
    for (int x = 0; x < CPW; ++x) {
      const uint32_t r = min(tile * BN + dr + 4 * x, kend - 1);
      dn_copy16(kg, r * rowb + 16 * ((lane & 15) ^ dn_swz(dr + 4 * x)), dst + 1024 * x);
    }
  };
  // V^T tile: 128 rows (dims) of 64 keys = 128 bytes; this wave fills rows 8(CPW w + x) + lane/8.
  // Its keys are the columns dn_vt_base(b) + 64 tile .. of the V^T rows (zeros past the sequence).
  const uint16_t* const vg = vt + (int64_t)g * 128 * tpad + dn_vt_base(seq0, b);
  const uint32_t vrowb = uint32_t(tpad) * 2;
  auto copy_v = [&](int stage, int tile) {
    const uint32_t dst = lds0 + kDnVst + stage * kDnTileB + 1024 * CPW * w;
#pragma unroll
    for (int x = 0; x < CPW; ++x) {
      const int d = 8 * (CPW * w + x) + (lane >> 3);
      dn_copy16(vg, d * vrowb + uint32_t(tile * BN) * 2 + 16 * ((lane & 7) ^ ((d >> 1) & 7)), dst + 1024 * x);
    }
  };

  // LDS operand addresses.  K: row kperm(qc) (+32 for keys 32..63), unit 2 s2 + hf, i.e. byte
  // kbase ^ 32 s2 with kbase = that row's unit-hf address.  V^T: row (dim) 32 db + qc, unit
  // 2 kq + hf (keys 16 kq + 8 hf ..), i.e. byte (vbase ^ 32 kq) + 4096 db.  Stage offsets are
  // added once per half step; half-tile and dim-block offsets are immediates.
  int kbase, vbase;
  {
    const int row = kperm(qc);
    kbase = kDnKst + 256 * row + 16 * (hf ^ dn_swz(row));
    const int sw = (qc >> 1) & 7;
    vbase = kDnVst + 128 * qc + 32 * (sw >> 1) + 16 * (hf ^ (sw & 1));
  }

  // S^T of one half tile (keys 32 hb ..) of the tile in K stage ks
  auto qk_half = [&](f32x16& s, int ks, int hb) {
    const int kb = kbase + ks * kDnTileB + 8192 * hb;
    s = (f32x16){};
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) s = mfma_bf16_32x32x16(dn_ld128(lb + (kb ^ (32 * s2))), qf[s2], s);
  };
  // P = fp16 of 2^(s scale - m): p[kk2] packs registers 8 kk2 .. 8 kk2 + 7 (8 consecutive keys,
  // the B operand of one PV k-step).  Returns the lane's sum of the fp16 P.
  const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
  auto expo = [&](const f32x16& s, i32x4 (&p)[2], float m) -> float {
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(fmaf(s[8 * kk2 + i], scale_log2, -m));
      const i32x4 pk = pack_f16x8(x);
      p[kk2] = pk;
      ps0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[0]), one, ps0, false);
      ps1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[1]), one, ps1, false);
      ps0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[2]), one, ps0, false);
      ps1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[3]), one, ps1, false);
    }
    return ps0 + ps1;
  };
  // row maxima of raw scores (both lane halves of a query column), in log2 units
  auto rowmax = [&](const f32x16& s) -> float {
    float mt = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[i]);
    return fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;
  };
  // causal mask of half hb of tile t: keys past the lane's query.  Register i holds key
  // 64t + 32hb + 8hf + c(i), c(i) = 16(i/8) + 4((i/4)%2) + i%4 (the kperm row order).
  auto mask = [&](f32x16& s, int t, int hb) {
    const int lim = my_q - BN * t - 32 * hb - 8 * hf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
      if (c > lim) s[i] = -__builtin_inff();
    }
  };

  // ---- prologue: Q, K(0), K(1), V(0) land; V stage 2 holds the pipeline's tile -1 (zeros, with
  // P(-1) = 0); S(0, keys 0..31) and the reference maxima from all of tile 0
  copy_k(0, 0);
  if (nt > 1) copy_k(1, 1);
  copy_v(0, 0);
  {
    i32x4* z = reinterpret_cast<i32x4*>(lds + kDnVst + 2 * kDnTileB) + CPW * tid;
#pragma unroll
    for (int x = 0; x < CPW; ++x) z[x] = (i32x4){0, 0, 0, 0};
  }
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) asm volatile("" : "+v"(qf[s2]));  // Q has landed
  dn_sync();

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16){};
  f32x16 sa, sb;       // scores: sa = S(t, keys 0..31), sb = S(t, keys 32..63)
  i32x4 pa[2], pb[2];  // probabilities: pa = P(t, keys 0..31), pb = P(t-1 or t, keys 32..63)
#pragma unroll
  for (int x = 0; x < 2; ++x) pb[x] = (i32x4){0, 0, 0, 0};
  float m_ref = 0.f, l_run = 0.f;
  if (wlast >= 0) {
    qk_half(sa, 0, 0);
    qk_half(sb, 0, 1);
    if (wlast == 0) {
      mask(sa, 0, 0);
      mask(sb, 0, 1);
    }
    const float mt = fmaxf(rowmax(sa), rowmax(sb));
    m_ref = (mt == -__builtin_inff()) ? 0.f : mt;
  }

  // One half step: 8 QK MFMAs into sn (K stage ks, keys 32 kh ..), 8 PV MFMAs with P = pv (V^T
  // stage vs, keys 32 vh ..), 16 exponentials of sc into pn with their row sums.  Operand reads
  // run two MFMAs of their kind ahead; packing and the row-sum term of element pair p come two
  // steps after its second exponential.
  auto half = [&](f32x16& sn, int ks, int kh, const i32x4 (&pv)[2], int vs, int vh, const f32x16& sc,
                  i32x4 (&pn)[2]) -> float {
    const int kb = kbase + ks * kDnTileB + 8192 * kh;      // K rows 32 kh ..
    const int vb = (vbase + vs * kDnTileB) ^ (64 * vh);    // V^T units 4 vh .. (keys 32 vh ..)
    __builtin_amdgcn_sched_barrier(0);
    i32x4 kop[8], vop[8];
    auto kread = [&](auto ii) {
      constexpr int i = decltype(ii)::value;
      kop[i] = dn_ld128(lb + (kb ^ (32 * i)));
    };
    auto vread = [&](auto ii) {  // PV MFMA i: k-step i/4 of the half, O block i%4
      constexpr int i = decltype(ii)::value;
      vop[i] = dn_ld128(lb + (vb ^ (32 * (i >> 2))) + 4096 * (i & 3));
    };
    kread(dn_ic<0>{});
    vread(dn_ic<0>{});
    kread(dn_ic<1>{});
    vread(dn_ic<1>{});
    float ps0 = 0.f, ps1 = 0.f, xe[4];
    auto pack = [&](auto pi) {  // fp16 pair of elements 2p, 2p+1 into pn, and its row-sum term
      constexpr int pr = decltype(pi)::value;
      const f16x2 h2 = {(_Float16)xe[2 * (pr & 1)], (_Float16)xe[2 * (pr & 1) + 1]};
      pn[pr >> 2][pr & 3] = __builtin_bit_cast(int, h2);
      if constexpr (pr & 1) ps1 = __builtin_amdgcn_fdot2(h2, one, ps1, false);
      else ps0 = __builtin_amdgcn_fdot2(h2, one, ps0, false);
    };
    auto step = [&](auto jj) {
      constexpr int jx = decltype(jj)::value, i = jx >> 1;
      if constexpr ((jx & 1) == 0) {
        if constexpr (i + 2 < 8) kread(dn_ic<i + 2>{});
        if constexpr (i == 0) sn = mfma_bf16_32x32x16(kop[0], qf[0], (f32x16){});
        else sn = mfma_bf16_32x32x16(kop[i], qf[i], sn);
      } else {
        if constexpr (i + 2 < 8) vread(dn_ic<i + 2>{});
        o[i & 3] = mfma_f16_32x32x16(vop[i], pv[i >> 2], o[i & 3]);
      }
      if constexpr ((jx & 1) == 0 && jx >= 4) pack(dn_ic<(jx >> 1) - 2>{});  // frees slot jx % 4
      xe[jx & 3] = __builtin_amdgcn_exp2f(fmaf(sc[jx], scale_log2, -m_ref));
      __builtin_amdgcn_sched_barrier(0);
    };
    step(dn_ic<0>{});
    step(dn_ic<1>{});
    step(dn_ic<2>{});
    step(dn_ic<3>{});
    step(dn_ic<4>{});
    step(dn_ic<5>{});
    step(dn_ic<6>{});
    step(dn_ic<7>{});
    step(dn_ic<8>{});
    step(dn_ic<9>{});
    step(dn_ic<10>{});
    step(dn_ic<11>{});
    step(dn_ic<12>{});
    step(dn_ic<13>{});
    step(dn_ic<14>{});
    step(dn_ic<15>{});
    pack(dn_ic<6>{});
    pack(dn_ic<7>{});
    return ps0 + ps1;
  };
  // lazy-reference check of the half just exponentiated (keys 32 hb .. of tile t, K stage ks)
  auto settle = [&](float ps, int t, int ks, int hb, i32x4 (&p)[2]) {
    if (__builtin_amdgcn_ballot_w64(!(ps <= 32768.f))) {
      // some P would leave fp16's range: recompute the half's scores, move the reference to the
      // row maxima, rescale O and l, redo its P
      f32x16 sr;
      qk_half(sr, ks, hb);
      if (t == wlast) mask(sr, t, hb);
      const float m_new = fmaxf(m_ref, rowmax(sr));
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_ref = m_new;
      ps = expo(sr, p, m_ref);
    }
    l_run += ps;
  };
  auto next3 = [](int x) { return x == 2 ? 0 : x + 1; };
  auto prev3 = [](int x) { return x == 0 ? 2 : x - 1; };
  // Iteration t (stage s = t % 3 of both rings): copies K(t+2) and V(t+1) into stage (t+2)%3 and
  // (t+1)%3, reads K(t), K(t+1), V(t-1), V(t); the barrier ending iteration t-1 has released both
  // stages written here.
  auto copies = [&](int t, int st) {
    if (t + 2 < nt) copy_k(prev3(st), t + 2);
    if (t + 1 < nt) copy_v(next3(st), t + 1);
  };
  int t = 0, st = 0;
  if (wlast >= 0) {
    for (; t <= wlast; ++t) {
      copies(t, st);
      if (t == wlast && t > 0) mask(sa, t, 0);
      // A: S(t, 32..63) | P(t, 0..31) | V(t-1, 32..63) P(t-1, 32..63)
      float ps = half(sb, st, 1, pb, prev3(st), 1, sa, pa);
      settle(ps, t, st, 0, pa);
      if (t == wlast) mask(sb, t, 1);
      // B: S(t+1, 0..31) | P(t, 32..63) | V(t, 0..31) P(t, 0..31)
      ps = half(sa, next3(st), 0, pa, st, 0, sb, pb);
      settle(ps, t, st, 1, pb);
      dn_sync();  // K(t+2) and V(t+1) have landed
      st = next3(st);
    }
    // iteration wlast + 1: the last half's P.V only
    copies(t, st);
    {
      const int vb = (vbase + prev3(st) * kDnTileB) ^ 64;  // keys 32..63
#pragma unroll
      for (int i = 0; i < 8; ++i)
        o[i & 3] = mfma_f16_32x32x16(dn_ld128(lb + (vb ^ (32 * (i >> 2))) + 4096 * (i & 3)), pb[i >> 2], o[i & 3]);
    }
    dn_sync();
    st = next3(st);
    ++t;
  }
  // the workgroup's remaining iterations: copies and barriers only
  for (; t <= nt; ++t) {
    copies(t, st);
    dn_sync();
    st = next3(st);
  }

  if (wlast < 0 || wq0 + qc >= kend) return;
  const float inv = 1.f / (l_run + __shfl_xor(l_run, 32));
  uint16_t* op = out + ((seq0 + wq0 + qc) * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dim = 32 * db + 8 * a + 4 * hf;
      uint32_t lo = f32_to_bf16(o[db][4 * a + 0] * inv) | (uint32_t(f32_to_bf16(o[db][4 * a + 1] * inv)) << 16);
      uint32_t hi = f32_to_bf16(o[db][4 * a + 2] * inv) | (uint32_t(f32_to_bf16(o[db][4 * a + 3] * inv)) << 16);
      *reinterpret_cast<uint2*>(op + dim) = make_uint2(lo, hi);
    }
}

// ------------------------------------------------------------------------------------------

hipError_t launch_gather_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int32_t* idx, int K, int mode, const int32_t* cu, int nseq,
                                   const int32_t* cache_lens, int cap, int64_t rows, int Hq, int Hkv,
                                   float scale, int keys_per_split, int nsplit, uint16_t* out,
                                   float* o_part, float2* ml_part, hipStream_t st, float* lse_out,
                                   const int32_t* order) {
  if (rows == 0) return hipSuccess;
  // 32-bit gather offsets: a key index (below its sequence's length <= rows, or below cap) times
  // Hkv x 128 x 2 bytes
  if ((uint64_t)(mode == 0 ? rows : cap) * Hkv * 128 * 2 > 0xFFFFFFFFull) return hipErrorInvalidValue;
  const float scale_log2 = scale * 1.4426950408889634f;
  if (mode == 0 && nsplit == 1 && idx && K <= kRowKeys && 8 % Hkv == 0) {
    constexpr int NWR = 4;
    const int64_t groups = (rows + NWR - 1) / NWR;
    const int hp = kGatherHeadsPerPhase < Hkv ? kGatherHeadsPerPhase : Hkv;  // heads gathered at once
    const int per = 8 / hp;  // XCDs per head
    const int64_t chunks = (groups + per * kGatherChunk - 1) / (per * kGatherChunk);
    const int64_t bpp = 8 * chunks * kGatherChunk;
    gather_rows_kernel<128, NWR><<<(unsigned)(bpp * (Hkv / hp)), 64 * NWR, 0, st>>>(
        q, k, v, idx, K, cu, nseq, rows, Hq, Hkv, scale_log2, out, lse_out, hp, (unsigned)bpp, order);
    return hipGetLastError();
  }
  dim3 grid((unsigned)rows, nsplit);
#define DSA_GATHER(NW)                                                                                   \
  gather_attention_kernel<128, NW><<<grid, 64 * NW, 0, st>>>(q, k, v, idx, K, mode, cu, nseq, cache_lens, \
                                                            cap, Hq, Hkv, scale_log2, keys_per_split,    \
                                                            nsplit, out, o_part, ml_part, lse_out)
  switch (Hkv) {
    case 1: DSA_GATHER(1); break;
    case 2: DSA_GATHER(2); break;
    case 3: DSA_GATHER(3); break;
    case 4: DSA_GATHER(4); break;
    case 5: DSA_GATHER(5); break;
    case 6: DSA_GATHER(6); break;
    case 7: DSA_GATHER(7); break;
    case 8: DSA_GATHER(8); break;
    default: return hipErrorInvalidValue;
  }
#undef DSA_GATHER
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nsplit == 1) return err;
  combine_kernel<<<dim3((unsigned)rows, Hq), 128, 0, st>>>(o_part, ml_part, nsplit, Hq, 128, out);
  return hipGetLastError();
}

// V^T in fp16 for the dense kernel's P.V MFMA, written once (exact for bf16 values in fp16's
// normal range) instead of by every workgroup that stages a key: vt[g][d][c] for KV head g and
// dim d, rows of tpad columns, sequence b from column dn_vt_base(b) (see there).

// One workgroup per 128-token block (b, j) of the dense schedule and KV head: two 64-token
// halves transposed through LDS.
__global__ __launch_bounds__(256) void v_transpose_kernel(const uint16_t* __restrict__ v, const int32_t* __restrict__ cu,
                                                          const int2* __restrict__ sched, const int* __restrict__ count,
                                                          int Hkv, int64_t tpad, uint16_t* __restrict__ vt) {
  __shared__ uint16_t tile[128][64 + 2];  // [dim][token], padded against bank conflicts
  if ((int)blockIdx.x >= *count) return;
  const int2 e = sched[blockIdx.x];
  const int b = e.x, g = blockIdx.y, tid = threadIdx.x;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  uint16_t* const rows = vt + (int64_t)g * 128 * tpad + dn_vt_base(seq0, b);
  for (int half = 0; half < 2; ++half) {
    const int i0 = 128 * e.y + 64 * half;  // first token of the half, relative to the sequence
    if (i0 >= L) break;
    if (half) __syncthreads();
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int u = tid + 256 * x, tt = u >> 4, d0 = 8 * (u & 15);  // token i0+tt, dims d0 .. d0+7
      float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (i0 + tt < L) {
        const i32x4 a =
            __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(v + ((seq0 + i0 + tt) * Hkv + g) * 128 + d0));
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = bf16_to_f32(bf16_lane(a, k));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) tile[d0 + k][tt] = __builtin_bit_cast(uint16_t, (_Float16)f[k]);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int u = tid + 256 * x, d = u >> 3, c = 8 * (u & 7);  // dim d, tokens i0+c .. i0+c+7
      if (i0 + c >= L) continue;
      i32x4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = int(uint32_t(tile[d][c + 2 * k]) | (uint32_t(tile[d][c + 2 * k + 1]) << 16));
      *reinterpret_cast<i32x4*>(rows + (int64_t)d * tpad + i0 + c) = w;  // columns past L: zeros
    }
  }
}

// The 64 zero columns after each sequence (columns L .. L+63 past its base; the transpose
// already wrote zeros up to the next multiple of 8), for every (KV head, dim) row.
__global__ __launch_bounds__(256) void v_pad_zero_kernel(const int32_t* __restrict__ cu, int nseq, int Hkv, int64_t tpad,
                                                         uint16_t* __restrict__ vt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (sequence, row, column 0..63)
  const int64_t rows = (int64_t)Hkv * 128;
  if (i >= nseq * rows * 64) return;
  const int b = int(i / (rows * 64));
  const int64_t r = (i / 64) % rows;
  const int col = int(i & 63);
  vt[r * tpad + dn_vt_base(cu[b], b) + (cu[b + 1] - cu[b]) + col] = 0;
}

// Columns of the V^T rows for T tokens in nseq sequences: the last sequence ends before
// round64(T) + 128 nseq + 64.
int64_t dense_vt_cols(int64_t T, int nseq) { return (T + 63) / 64 * 64 + 128 * (int64_t(nseq) + 1); }

// vt: Hkv * 128 * dense_vt_cols(T, nseq) halves of scratch for V^T in fp16.
hipError_t launch_dense_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* vt, int64_t T,
                                const int32_t* cu, int nseq, int Hq, int Hkv, float scale, const int2* sched,
                                const int* count, int nb_bound, uint16_t* out, hipStream_t st) {
  if (nb_bound == 0) return hipSuccess;
  const int64_t tpad = dense_vt_cols(T, nseq);
  // 32-bit copy offsets within a KV head's K rows and V^T rows
  if ((uint64_t)T * Hkv * 128 * 2 > 0xFFFFFFFFull || (uint64_t)tpad * 128 * 2 > 0xFFFFFFFFull)
    return hipErrorInvalidValue;
  v_transpose_kernel<<<dim3(nb_bound, Hkv), 256, 0, st>>>(v, cu, sched, count, Hkv, tpad, vt);
  const int64_t pads = (int64_t)nseq * Hkv * 128 * 64;
  v_pad_zero_kernel<<<(unsigned)((pads + 255) / 256), 256, 0, st>>>(cu, nseq, Hkv, tpad, vt);
  const float sl2 = scale * 1.4426950408889634f;
  if ((Hq / Hkv) % 2 == 0)
    dense_prefill_kernel<2><<<dim3(nb_bound, Hq / 2), 512, 0, st>>>(q, k, vt, tpad, cu, Hq, Hkv, sl2, sched, count, out);
  else
    dense_prefill_kernel<1><<<dim3(nb_bound, Hq), 256, 0, st>>>(q, k, vt, tpad, cu, Hq, Hkv, sl2, sched, count, out);
  return hipGetLastError();
}

}  // namespace dsa
