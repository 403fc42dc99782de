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
//   128 query tokens x 2 query heads of one KV group; 64-key K/V tiles are double-buffered in
//   LDS and shared by both heads; S^T and O^T use 32x32x16 MFMAs (bf16 for QK, fp16 for PV,
//   with V converted to fp16 once beforehand).
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
    auto issue = [&](VTile& t, int tl) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const i32x4 sk = *reinterpret_cast<const i32x4*>(il + tl + 8 * (lr >> 2) + 4 * h);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          __builtin_amdgcn_global_load_lds(kg_base + (int64_t)max(sk[c], 0) * kvs + 32 * lg + 8 * (lr & 3),
                                           kb + (4 * h + c) * kKRegion, 16, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the K loads ahead of the V loads (vmcnt order)
      const i32x4 s0 = *reinterpret_cast<const i32x4*>(il + tl + 8 * lg);
      const i32x4 s1 = *reinterpret_cast<const i32x4*>(il + tl + 8 * lg + 4);
#pragma unroll
      for (int m = 0; m < 4; ++m) { t.sv[m] = s0[m]; t.sv[4 + m] = s1[m]; }
#pragma unroll
      for (int m = 0; m < 8; ++m)
        t.vf[m] = *reinterpret_cast<const i32x4*>(vg_base + (int64_t)max(t.sv[m], 0) * kvs + 8 * lr);
    };
    const __attribute__((address_space(3))) uint8_t* kr = kb + (lr & 3) * kKRegion + (4 * (lr >> 2) + 16 * lg) * 16;
    VTile vc, vn;
    if (cnt32 > 0) issue(vc, 0);
    for (int tl = 0; tl < cnt32; tl += 32) {
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
        issue(vn, tl + 32);
      }
      compute(kf, vc.vf, vc.sv);
      vc = vn;
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
__global__ __launch_bounds__(64 * NW) void gather_attention_kernel(
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
  const int g = threadIdx.x >> 6;
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
__global__ __launch_bounds__(64 * NW) void gather_rows_kernel(
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
  const int wave = threadIdx.x >> 6;
  const int64_t rslot = group * NW + wave;
  if (rslot >= rows) return;  // waves are independent: no workgroup barrier below
  const int64_t r = order ? (int64_t)order[rslot] : rslot;  // the row this slot serves
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
// Workgroup = 8 waves: 128 query tokens x 2 query heads of one KV group (waves 0-3 head 2p,
// waves 4-7 head 2p+1, 32 tokens each), so every K/V tile staged in LDS serves both heads.
// K/V tiles of 64 keys are double-buffered: the next tile is loaded into registers while the
// current one is computed, then written to the other LDS buffer; one barrier per tile.
// MFMA operand layouts and the kperm / transposed-read scheme: attn_tiles.h.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(512) void dense_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu, int Hq, int Hkv, float scale_log2, const int2* __restrict__ sched,
    const int* __restrict__ sched_count, int pair, uint16_t* __restrict__ out) {
  constexpr int D = 128, BM = 128, BN = 64;
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2][2][kKvTileB];  // [buffer][K=0/V=1]
  const int n = blockIdx.x;
  if (n >= *sched_count) return;
  const int2 e = sched[n];
  const int b = e.x, j = e.y;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // pair != 0: waves 0-3 take head 2y, waves 4-7 head 2y+1 (same KV head since G is even);
  // pair == 0 (odd G): one head per workgroup, waves 4-7 only help stage the tiles
  const int h = pair ? 2 * blockIdx.y + (w >> 2) : blockIdx.y;
  const bool active = pair || w < 4;
  const int g = h / G;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int q0 = BM * j;
  const int rows = min(BM, L - q0);
  const int kend = q0 + rows;
  const int qc = lane & 31, hf = lane >> 5;
  const int64_t kvs = (int64_t)Hkv * D;
  const int my_q = q0 + 32 * (w & 3) + qc;

  i32x4 qf[8];
  {
    const int qq = min(my_q, kend - 1);
    const uint16_t* qp = q + ((seq0 + qq) * Hq + h) * D + 8 * hf;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) qf[s2] = *reinterpret_cast<const i32x4*>(qp + 16 * s2);
  }
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;
  const int wave_qmax = q0 + 32 * (w & 3) + 31;

  // tile loader: 512 threads x (2 K + 2 V) 16-byte units = 64 keys x 256 B each
  i32x4 pre[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int u = tid + 512 * x;  // unit 0..1023: key = u >> 4, 16-byte column c = u & 15
      const int kk = min(kt + (u >> 4), kend - 1);
      pre[x] = *reinterpret_cast<const i32x4*>(k + (seq0 + kk) * kvs + g * D + 8 * (u & 15));
      pre[2 + x] = *reinterpret_cast<const i32x4*>(v + (seq0 + kk) * kvs + g * D + 8 * (u & 15));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int u = tid + 512 * x;
      const int off = kv_off(u >> 4, 16 * (u & 15));
      *reinterpret_cast<i32x4*>(&kv_lds[buf][0][off]) = pre[x];
      *reinterpret_cast<i32x4*>(&kv_lds[buf][1][off]) = pre[2 + x];  // V already fp16
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int kt = 0; kt < kend; kt += BN) {
    const bool more = kt + BN < kend;
    if (more) gload(kt + BN);
    if (active && kt <= wave_qmax) {
      const uint8_t* kl = kv_lds[buf][0];
      const uint8_t* vl = kv_lds[buf][1];
      // S^T for two 32-key blocks
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
      // mask + scale; C row (reg i, half hf) of block rb <-> key kt + 32rb + kperm(8(i/4)+4hf+i%4).
      // Tiles wholly before the wave's first query need no mask (all but the last one or two).
      // The max is taken on the raw scores (the scale is positive) and the scale applied once
      // per element inside the exponent's fma.
      float z[2][16];
      float mt = -__builtin_inff();
      if (kt + BN - 1 <= q0 + 32 * (w & 3)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            z[rb][i] = sacc[rb][i];
            mt = fmaxf(mt, z[rb][i]);
          }
      } else {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt + 32 * rb + kperm(8 * (i >> 2) + 4 * hf + (i & 3));
            const float zz = (key <= my_q) ? sacc[rb][i] : -__builtin_inff();
            z[rb][i] = zz;
            mt = fmaxf(mt, zz);
          }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;
      // lazy reference max: it moves only when the query's tile max passes it by more than 8
      // (log2 units), so P <= 2^8 (exact enough in fp16) and the O rescale -- a round trip of
      // the accumulators through VALU -- happens on few tiles
      const bool move = mt > m_run + 8.f;  // false while every key so far is masked
      if (__ballot(move)) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;  // m_run = -inf: 0
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
        m_run = move ? mt : m_run;
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
      // O^T += V^T P^T; k-step (rb, kk2) covers keys 32rb + 16kk2 + 0..15 = registers 8kk2..8kk2+7
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
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!active || my_q >= kend) return;
  const float inv = 1.f / l_tot;
  uint16_t* op = out + ((seq0 + my_q) * Hq + h) * D;
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

// V converted to fp16 once (exact for bf16 values in fp16's normal range) for the fp16 P.V MFMA
// of the dense kernel, instead of once per staging workgroup (each key's V is staged by every
// later 128-query block of its sequence).
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t* __restrict__ in,
                                                          uint16_t* __restrict__ out, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const i32x4 x = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(in) + i);
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = bf16_to_f32(bf16_lane(x, e));
  reinterpret_cast<i32x4*>(out)[i] = pack_f16x8(f);
}

// v16: T * Hkv * 128 halves of scratch for V in fp16.
hipError_t launch_dense_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* v16, int64_t T,
                                const int32_t* cu, int Hq, int Hkv, float scale, const int2* sched, const int* count,
                                int nb_bound, uint16_t* out, hipStream_t st) {
  if (nb_bound == 0) return hipSuccess;
  const int64_t n8 = T * Hkv * 128 / 8;
  bf16_to_f16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(v, v16, n8);
  const int pair = ((Hq / Hkv) % 2 == 0) ? 1 : 0;
  dense_prefill_kernel<<<dim3(nb_bound, pair ? Hq / 2 : Hq), 512, 0, st>>>(
      q, k, v16, cu, Hq, Hkv, scale * 1.4426950408889634f, sched, count, pair, out);
  return hipGetLastError();
}

}  // namespace dsa
