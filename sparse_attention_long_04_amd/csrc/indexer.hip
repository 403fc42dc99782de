// Lightning Indexer scores for packed prefill (Keye-VL-2.0 summary page, gsyq.cn, section 一:
// one MQA-shared indexer key per position, scored by every indexer head):
//
//     I[t, s] = sum_h w[t, h] * max(0, q_I[t, h, :] . k_I[s, :]),   s <= t in t's sequence.
//
// Work unit: one workgroup owns a block of 16 query tokens of one sequence and sweeps all of
// their causal keys.  The block's indexer queries (16 tokens x H_I heads x d_I) sit in LDS;
// each wave streams 16-key tiles of k_I from HBM/L2 straight into MFMA operand registers.
// For every head, q_h (16 tokens) x k (16 keys) is ONE dense MFMA contraction over d_I
// (fp8: v_mfma_f32_16x16x128_f8f6f4; bf16: 16x16x32 steps); ReLU and the head weight are
// applied to the fp32 accumulator in registers and summed over heads without leaving VGPRs.
//
// Scores go to a triangle of 16-row blocks: block j of a sequence holds rows 16j..16j+15 with
// a row stride of 16(j+1) floats, at offset seqoff[b] + 128 j (j+1).
#include "common.h"

namespace dsa {

// ------------------------------------------------------------------------------------------
// Work schedule: (sequence, block) pairs of BQ query rows, longest (largest block index) first.
// Also writes seqoff[b] = start of sequence b's score triangle (16-row blocks, in floats).
// ------------------------------------------------------------------------------------------
__global__ void build_schedule_kernel(const int32_t* __restrict__ cu, int nseq, int bq,
                                      int nb_bound, int2* __restrict__ sched,
                                      int* __restrict__ sched_count, int64_t* __restrict__ seqoff) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (seqoff != nullptr && n <= nseq) {
    int64_t off = 0;
    for (int b = 0; b < n; ++b) {
      const int64_t nb16 = (cu[b + 1] - cu[b] + 15) / 16;
      off += 128 * nb16 * (nb16 + 1);
    }
    seqoff[n] = off;
  }
  if (n >= nb_bound) return;
  int acc = 0, b = -1, j = 0;
  for (int s = 0; s < nseq; ++s) {
    const int nb = (cu[s + 1] - cu[s] + bq - 1) / bq;
    if (b < 0 && n < acc + nb) { b = s; j = n - acc; }
    acc += nb;
  }
  if (n == 0) *sched_count = acc;
  if (b < 0) return;
  // rank in the order (block index descending, sequence ascending)
  int rank = 0;
  for (int s = 0; s < nseq; ++s) {
    const int nb = (cu[s + 1] - cu[s] + bq - 1) / bq;
    if (nb > j + 1) rank += nb - j - 1;
    if (s < b && nb > j) rank += 1;
  }
  sched[rank] = make_int2(b, j);
}

// ------------------------------------------------------------------------------------------
// Exact helpers for OCP e4m3 ("fn") values.
// ------------------------------------------------------------------------------------------

// Round to the e4m3 grid (nearest even), |result| <= 448.
__device__ __forceinline__ float e4m3_round(float v) {
  const float a = fabsf(v);
  const int ex = max(int((__float_as_uint(a) >> 23) & 0xFF) - 127, -6);
  const float qu = __uint_as_float(uint32_t(ex - 3 + 127) << 23);  // spacing of the grid at |v|
  const float r = fminf(rintf(a / qu) * qu, 448.f);
  return copysignf(r, v);
}

// Code of a value that lies on the e4m3 grid.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = uint32_t(a * 512.f);
  } else {
    const uint32_t bits = __float_as_uint(a);
    code = ((((bits >> 23) & 0xFFu) - 120u) << 3) | ((bits >> 20) & 7u);
  }
  return code | ((__float_as_uint(v) >> 24) & 0x80u);
}

// ------------------------------------------------------------------------------------------
// Indexer kernel.
//   FP8 = true : e4m3fn inputs, DI = 128, one 16x16x128 MFMA per (head, key tile).
//   FP8 = false: bf16 inputs, DI = 64 or 128, DI/32 16x16x32 MFMAs per (head, key tile).
// Lane layout (16x16 MFMA): lane l -> r = l & 15, g = l >> 4.  A (queries) lane holds token
// row r, B (keys) lane holds key r; both take bytes [g*CH, (g+1)*CH) of their d_I row, so
// every MFMA pairs identical d_I positions.  Output C[i] of lane l = (token 4g+i, key r).
//
// ReLU without a max per element: with c_h = q_h . k,
//     sum_h w_h relu(c_h) = ( sum_h w_h c_h  +  sum_h w_h |c_h| ) / 2 ,
// the |c_h| sum is one FMA per element (|.| is a free source modifier), and the linear sum is
// (sum_h w_h q_h) . k -- a per-token vector q_lin, split into NP pieces on the input grid
// (e4m3 pieces scaled by a power of two per block, or bf16 pieces) and contracted by NP extra
// MFMAs accumulating in place.  The halving is folded into the staged weights (w/2 is exact,
// and q_lin and its pieces then halve exactly).  For integer-valued inputs and power-of-two
// weights every quantity is a multiple of 1/16 below 2^17, so the result is exact in any
// summation order; otherwise the linear term carries about 20 (fp8) or 24 (bf16) significant
// bits.
// ------------------------------------------------------------------------------------------
template <bool FP8, int DI, int HMAX, int NWAVES, int NT>
__global__ __launch_bounds__(NWAVES * 64) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ w_idx, const int32_t* __restrict__ cu, int H,
    const int2* __restrict__ sched, const int* __restrict__ sched_count, int n0,
    const int64_t* __restrict__ seqoff, int64_t slot_stride, float* __restrict__ scores,
    float2* __restrict__ rowrange) {
  constexpr int ROWB = DI * (FP8 ? 1 : 2);   // bytes of one d_I row
  constexpr int UNITS = ROWB / 16;           // 16-byte units per row
  constexpr int CH = ROWB / 4;               // bytes per lane group
  constexpr int CHU = CH / 16;               // 16-byte units per lane group
  constexpr int NP = FP8 ? 5 : 3;            // pieces of q_lin
  constexpr int EPU = FP8 ? 16 : 8;          // elements per 16-byte unit
  static_assert(UNITS >= 8, "swizzle needs >= 8 units per row");
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[(HMAX + NP) * 16 * ROWB];
  // two heads of padding: the head loop's last reloads read (unused) heads H and H+1
  __shared__ __attribute__((aligned(16))) float w_lds[(HMAX + 2) * 16];
  __shared__ float2 range_lds[NWAVES][16];
  __shared__ uint32_t qmax_lds;
  __shared__ float scale_lds;
  // q_lin pieces follow head H-1 directly: the head loop's last reloads (heads H, H+1) then
  // fetch pieces 0 and 1
  uint8_t* const lin_lds = q_lds + H * 16 * ROWB;
  // 16-byte unit swizzle of row t (0..15) of a head's 16-row tile: an A-operand read (16 lanes =
  // 16 rows per 256-byte LDS pass) then touches 16 distinct bank groups.  128-byte rows pair up
  // in a pass, so rows t and t + 8 (same parity, same t & 7) need different units.
  auto swz = [](int t) { return UNITS == 8 ? ((t & 7) ^ ((t >> 3) & 1)) : (t & 15); };

  const int n = n0 + blockIdx.x;
  const int N = *sched_count;
  if (n >= N) return;
  // triangle mode: schedule order; chunk mode: the chunked loop's order
  const int2 e = sched[seqoff ? n : chunk_entry(n, N)];
  const int b = e.x, j = e.y;
  const int64_t seq0 = cu[b];
  const int L = cu[b + 1] - cu[b];
  const int i0 = 16 * j;
  const int rows = min(16, L - i0);
  const int kend = i0 + rows;  // keys [0, kend) are needed by this block
  const int tid = threadIdx.x;

  // stage queries: lds[(h*16 + t)*ROWB + ((c ^ swz(t)) * 16)] <- q_idx[seq0+i0+t][h][c*16..].
  // The block's H*ROWB-byte token rows are contiguous, so 16-byte unit u sits at base + 16u.
  // Every load is issued before the first store (addresses clamped to the block's rows, rows
  // past the end stored as zeros): one round trip instead of one per unit.
  {
    constexpr int NT_ = NWAVES * 64;
    constexpr int SPT = (16 * HMAX * UNITS + NT_ - 1) / NT_;  // units per thread
    constexpr int WPT = (16 * HMAX + NT_ - 1) / NT_;          // weights per thread
    const int per_tok = H * UNITS;
    const int total = 16 * per_tok, valid = rows * per_tok;
    const i32x4* qsrc = reinterpret_cast<const i32x4*>(q_idx + (seq0 + i0) * H * (int64_t)ROWB);
    i32x4 sv[SPT];
    float wsv[WPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) sv[k] = __builtin_nontemporal_load(qsrc + min(tid + k * NT_, valid - 1));
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int u = tid + k * NT_;
      const int h = min(u >> 4, H - 1), t = min(u & 15, rows - 1);
      wsv[k] = w_idx[(seq0 + i0 + t) * H + h];
    }
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int u = tid + k * NT_;
      if (u < total) {
        const int t = u / per_tok;
        const int rem = u - t * per_tok;
        const int h = rem / UNITS;
        const int c = rem - h * UNITS;
        const i32x4 zero = {0, 0, 0, 0};
        *reinterpret_cast<i32x4*>(q_lds + (h * 16 + t) * ROWB + ((c ^ swz(t)) * 16)) = u < valid ? sv[k] : zero;
      }
    }
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int u = tid + k * NT_;
      if (u < 16 * H) w_lds[u] = ((u & 15) < rows) ? 0.5f * wsv[k] : 0.f;  // the ReLU identity's 1/2
    }
    if (tid == 0) qmax_lds = 0u;
  }
  __syncthreads();

  // q_lin[t, :] = sum_h w[t,h] q[t,h,:]  (fp32, fixed head order), then its pieces
  {
    const bool act = tid < 16 * UNITS;
    const int t = tid / UNITS, u = tid - (tid / UNITS) * UNITS;
    float lin[EPU];
#pragma unroll
    for (int x = 0; x < EPU; ++x) lin[x] = 0.f;
    if (act) {
#pragma unroll 4
      for (int h = 0; h < H; ++h) {  // H is a multiple of 16
        const i32x4 val = *reinterpret_cast<const i32x4*>(q_lds + (h * 16 + t) * ROWB + ((u ^ swz(t)) * 16));
        const float wv = w_lds[h * 16 + t];
        if constexpr (FP8) {
          // the hardware's e4m3 -> fp32 pair conversion (exact): two codes per instruction
#pragma unroll
          for (int wd = 0; wd < 4; ++wd) {
            typedef float f32x2_t __attribute__((ext_vector_type(2)));
            const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(val[wd], false);
            const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(val[wd], true);
            lin[4 * wd + 0] = fmaf(wv, lo.x, lin[4 * wd + 0]);
            lin[4 * wd + 1] = fmaf(wv, lo.y, lin[4 * wd + 1]);
            lin[4 * wd + 2] = fmaf(wv, hi.x, lin[4 * wd + 2]);
            lin[4 * wd + 3] = fmaf(wv, hi.y, lin[4 * wd + 3]);
          }
        } else {
#pragma unroll
          for (int x = 0; x < EPU; ++x) {
            const uint32_t word = uint32_t(val[x / (EPU / 4)]);
            lin[x] = fmaf(wv, bf16_to_f32(uint16_t((x & 1) ? (word >> 16) : (word & 0xFFFFu))), lin[x]);
          }
        }
      }
    }
    float scale = 1.f;  // q_lin is contracted as sum_p piece_p * scale
    if constexpr (FP8) {
      float mx = 0.f;
#pragma unroll
      for (int x = 0; x < EPU; ++x) mx = fmaxf(mx, fabsf(lin[x]));
      if (act) atomicMax(&qmax_lds, __float_as_uint(mx));
      __syncthreads();
      // power of two S with max|q_lin| / S in (64, 240]: the block's largest entries use the top
      // of the e4m3 range (max 448) and small entries stay clear of its subnormal floor
      const float qm = __uint_as_float(qmax_lds);
      int es = 0;
      if (qm > 0.f) {
        es = int((__float_as_uint(qm) >> 23) & 0xFF) - 127 - 7;
        if (qm > 240.f * __uint_as_float(uint32_t(127 + max(es, -126)) << 23)) ++es;
        es = max(-100, min(100, es));
      }
      scale = __uint_as_float(uint32_t(127 + es) << 23);
      const float inv = __uint_as_float(uint32_t(127 - es) << 23);
#pragma unroll
      for (int x = 0; x < EPU; ++x) lin[x] *= inv;
    }
    if (act) {
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        i32x4 codes = {0, 0, 0, 0};
#pragma unroll
        for (int x = 0; x < EPU; ++x) {
          uint32_t c;
          float piece;
          if constexpr (FP8) {
            piece = e4m3_round(lin[x]);
            c = e4m3_encode(piece) << (8 * (x & 3));
          } else {
            const uint16_t hb = f32_to_bf16(lin[x]);
            piece = bf16_to_f32(hb);
            c = uint32_t(hb) << (16 * (x & 1));
          }
          lin[x] -= piece;
          codes[x / (EPU / 4)] |= int(c);
        }
        *reinterpret_cast<i32x4*>(lin_lds + (pc * 16 + t) * ROWB + ((u ^ swz(t)) * 16)) = codes;
      }
    }
    if (tid == 0) scale_lds = scale;
  }
  __syncthreads();
  const float lin_scale = scale_lds;

  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t stride = 16 * (int64_t)(j + 1);
  // the block's scores: in its sequence's triangle, or in slot blockIdx.x of a chunk buffer
  float* __restrict__ sblk = seqoff ? scores + seqoff[b] + score_block_offset(j)
                                    : scores + (int64_t)blockIdx.x * slot_stride;
  float rmin[4], rmax[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { rmin[i] = __builtin_inff(); rmax[i] = -__builtin_inff(); }

  auto load_b = [&](i32x4 (&dst)[NT][CHU], int kb) {
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      const int key = min(kb + 16 * jt + r, kend - 1);
      const uint8_t* p = k_idx + (seq0 + key) * (int64_t)ROWB + g * CH;
#pragma unroll
      for (int c = 0; c < CHU; ++c) dst[jt][c] = *reinterpret_cast<const i32x4*>(p + 16 * c);
    }
  };
  auto mma = [&](const i32x4 (&a)[CHU], const i32x4 (&bb)[CHU], f32x4 c) -> f32x4 {
    if constexpr (FP8) {
      const i32x8 a8 = {a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
      const i32x8 b8 = {bb[0][0], bb[0][1], bb[0][2], bb[0][3], bb[1][0], bb[1][1], bb[1][2], bb[1][3]};
      return mfma_fp8_16x16x128(a8, b8, c);
    } else {
#pragma unroll
      for (int cc = 0; cc < CHU; ++cc) c = mfma_bf16_16x16x32(a[cc], bb[cc], c);
      return c;
    }
  };
  auto load_a = [&](i32x4 (&dst)[CHU], const uint8_t* base) {
    const uint8_t* qa = base + r * ROWB;
#pragma unroll
    for (int c = 0; c < CHU; ++c) dst[c] = *reinterpret_cast<const i32x4*>(qa + (((g * CHU + c) ^ swz(r)) * 16));
  };

  constexpr int STEP = NWAVES * NT * 16;
  // one wave step over NT key tiles; the next step's tiles are loaded into the other buffer
  // (ping-pong, no register copies, so the loads stay in flight across the head loop)
  auto kb_body = [&](const i32x4 (&cur)[NT][CHU], i32x4 (&nxt)[NT][CHU], int kb) {
    // unconditional (addresses are clamped): a fixed number of loads in flight lets the
    // compiler wait only for the current buffer
    load_b(nxt, kb + STEP);
    f32x4 acc_abs[NT], acc_lin[NT];  // acc_abs: first written by the first step's fold
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) acc_lin[jt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // Software pipeline over head pairs (H is a multiple of 16, so the pair count P = H/2 is
    // even).  c0/c1 hold the previous pair's products while this pair's MFMAs run: each MFMA is
    // preceded by the four FMAs that fold the product it will overwrite, so the VALU work
    // co-issues with the matrix pipe.  A head's A registers are reloaded (for the head two
    // further on) as soon as its last MFMA has issued, so the LDS read has four MFMAs of time to
    // land.  Head weights sit in two slots, even pairs in wx, odd pairs in wy: a step folds
    // with one slot and then reloads it for the pair two ahead, so no register copies (which
    // would wait on the fresh loads) are needed.  The scheduling barriers keep the compiler
    // from hoisting the FMAs or the reloads out of this order.
    f32x4 c0[NT], c1[NT];
    i32x4 a0[CHU], a1[CHU];
    auto w4 = [&](int h) { return *reinterpret_cast<const f32x4*>(w_lds + h * 16 + 4 * g); };
    load_a(a0, q_lds);
    load_a(a1, q_lds + 16 * ROWB);
    f32x4 wx0 = w4(0), wx1 = w4(1);
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) c0[jt] = mma(a0, cur[jt], (f32x4){0.f, 0.f, 0.f, 0.f});
    __builtin_amdgcn_sched_barrier(0);
    load_a(a0, q_lds + 2 * 16 * ROWB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) c1[jt] = mma(a1, cur[jt], (f32x4){0.f, 0.f, 0.f, 0.f});
    __builtin_amdgcn_sched_barrier(0);
    load_a(a1, q_lds + 3 * 16 * ROWB);
    f32x4 wy0 = w4(2), wy1 = w4(3);
    __builtin_amdgcn_sched_barrier(0);
    // step for the pair of heads h, h+1 (a0/a1 in flight); folds pair h-2 with (wf0, wf1)
    auto step = [&](f32x4& wf0, f32x4& wf1, int h, bool first) {
      // the last step reloads "heads" H, H+1 = q_lin pieces 0 and 1 (their weights, read from
      // w_lds's padding, are never used)
      const int hq = h + 2;
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc_abs[jt][i] = first ? wf0[i] * fabsf(c0[jt][i]) : fmaf(wf0[i], fabsf(c0[jt][i]), acc_abs[jt][i]);
        c0[jt] = mma(a0, cur[jt], (f32x4){0.f, 0.f, 0.f, 0.f});
        __builtin_amdgcn_sched_barrier(0);
      }
      load_a(a0, q_lds + hq * 16 * ROWB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_abs[jt][i] = fmaf(wf1[i], fabsf(c1[jt][i]), acc_abs[jt][i]);
        c1[jt] = mma(a1, cur[jt], (f32x4){0.f, 0.f, 0.f, 0.f});
        __builtin_amdgcn_sched_barrier(0);
      }
      load_a(a1, q_lds + (hq + 1) * 16 * ROWB);
      wf0 = w4(hq);
      wf1 = w4(hq + 1);
      __builtin_amdgcn_sched_barrier(0);
    };
    // step p folds pair p-1: odd p with wx (even pairs' weights), even p with wy
    step(wx0, wx1, 2, true);
    for (int h = 4; h < H; h += 4) {  // pairs 2 .. P-1, two per iteration
      step(wy0, wy1, h, false);
      step(wx0, wx1, h + 2, false);
    }
    // q_lin . k: NP pieces (0 and 1 already in a0/a1, in flight), each reloaded register set
    // fetching the piece two further on; the last pair's fold co-issues with piece 0
#pragma unroll
    for (int pc = 0; pc < NP; ++pc) {
      i32x4(&a)[CHU] = (pc & 1) ? a1 : a0;
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        if (pc == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc_abs[jt][i] = fmaf(wy0[i], fabsf(c0[jt][i]), acc_abs[jt][i]);
            acc_abs[jt][i] = fmaf(wy1[i], fabsf(c1[jt][i]), acc_abs[jt][i]);
          }
        }
        acc_lin[jt] = mma(a, cur[jt], acc_lin[jt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (pc + 2 < NP) load_a(a, lin_lds + (pc + 2) * 16 * ROWB);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (rows == 16 && kb + NT * 16 <= i0 + 1) {
      // every (row, key) of this step is causal: no masking
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        const int key = kb + 16 * jt + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = fmaf(acc_lin[jt][i], lin_scale, acc_abs[jt][i]);
          sblk[(4 * g + i) * stride + key] = v;
          rmin[i] = fminf(rmin[i], v);
          rmax[i] = fmaxf(rmax[i], v);
        }
      }
    } else {
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        const int key = kb + 16 * jt + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * g + i;
          const float v = fmaf(acc_lin[jt][i], lin_scale, acc_abs[jt][i]);
          if (row < rows && key <= i0 + row) {
            sblk[row * stride + key] = v;
            rmin[i] = fminf(rmin[i], v);
            rmax[i] = fmaxf(rmax[i], v);
          }
        }
      }
    }
  };
  i32x4 bA[NT][CHU], bB[NT][CHU];
  const int kb0 = wave * NT * 16;
  if (kb0 < kend) load_b(bA, kb0);
  for (int kb = kb0; kb < kend; kb += 2 * STEP) {
    kb_body(bA, bB, kb);
    if (kb + STEP < kend) kb_body(bB, bA, kb + STEP);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      rmin[i] = fminf(rmin[i], __shfl_xor(rmin[i], o));
      rmax[i] = fmaxf(rmax[i], __shfl_xor(rmax[i], o));
    }
    if (r == 0) range_lds[wave][4 * g + i] = make_float2(rmin[i], rmax[i]);
  }
  __syncthreads();
  if (tid < rows) {
    float2 acc2 = range_lds[0][tid];
    for (int w = 1; w < NWAVES; ++w) {
      acc2.x = fminf(acc2.x, range_lds[w][tid].x);
      acc2.y = fmaxf(acc2.y, range_lds[w][tid].y);
    }
    rowrange[seq0 + i0 + tid] = acc2;
  }
}

// Expand the rows of one chunk of 16-row blocks (slot c of the chunk buffer holds the block at
// position n0 + c of the chunked loop, schedule entry chunk_entry(n0 + c), rows with a stride of
// 16(j+1) floats) into a dense [T, ldo] matrix, -inf outside the
// causal context.  One workgroup per (slot, row).
__global__ void unpack_scores_kernel(const float* __restrict__ buf, int64_t slot_stride,
                                     const int2* __restrict__ sched, const int* __restrict__ sched_count,
                                     int n0, const int32_t* __restrict__ cu, int ldo, float* __restrict__ out) {
  const int slot = blockIdx.x >> 4, rr = blockIdx.x & 15;
  const int n = n0 + slot;
  const int N = *sched_count;
  if (n >= N) return;
  const int2 e = sched[chunk_entry(n, N)];
  const int b = e.x, j = e.y, i = 16 * j + rr;
  if (i >= cu[b + 1] - cu[b]) return;
  const int64_t t = cu[b] + i;
  const float* src = buf + (int64_t)slot * slot_stride + (int64_t)rr * 16 * (j + 1);
  for (int s = threadIdx.x; s < ldo; s += blockDim.x)
    out[t * ldo + s] = (s <= i) ? src[s] : -__builtin_inff();
}

// ------------------------------------------------------------------------------------------
// Decode indexer: one query token per sequence against its whole cache.  A = the token's
// queries (16 heads per MFMA, from LDS), B = 16 cached keys; C[i] of lane l = (head 4g+i,
// key r).  The weighted ReLU sum over heads runs in registers, then across the 4 lane groups.
// Each workgroup (kDecodeKeysPerBlock keys) writes its scores as order keys sorted by selection bin
// (key >> kDecodeBinShift), highest bin first: skeys[b][blk][slot] and their positions inside the
// block spos[b][blk][slot] (8 bits), the keys below its histogram window last.  It also writes the
// window itself: wbase[b][blk] = decode_win_base of its largest key and wcnt[b][blk][i] = the
// number of its keys in bins wbase + i and above (cumulative 16-bit counts, kDecodeWinBins bins;
// keys below the window are not counted).  All plain stores: the
// selection needs nothing cleared beforehand.  The bin sort is a counting sort: a key's rank in
// its bin is the value its histogram atomic returned.
// ------------------------------------------------------------------------------------------
template <int HMAX, int NT>
__global__ __launch_bounds__(256) void indexer_decode_kernel(
    const uint8_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_cache, const int32_t* __restrict__ cache_lens, int cap, int H,
    uint32_t* __restrict__ skeys, uint8_t* __restrict__ spos, int* __restrict__ wbase, uint16_t* __restrict__ wcnt,
    int blk_stride) {
  constexpr int ROWB = 128, UNITS = 8;
  constexpr int WKEYS = kDecodeKeysPerBlock / 4;  // contiguous keys per wave
  static_assert(WKEYS == 2 * NT * 16, "a wave's keys are two steps of NT tiles");
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[HMAX * ROWB];
  __shared__ float w_lds[HMAX];
  __shared__ uint32_t red_lds[4];
  __shared__ int win_lds[kDecodeWinBins + 1];   // [kDecodeWinBins]: keys below the window
  __shared__ int off_lds[kDecodeWinBins + 1];
  const int b = blockIdx.y;
  const int n = cache_lens[b];
  const int key0 = blockIdx.x * kDecodeKeysPerBlock;
  const int tid = threadIdx.x;
  if (key0 >= n) return;
  const int wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  if (tid <= kDecodeWinBins) win_lds[tid] = 0;
  // 16-byte unit swizzle of head row h: the 16 heads an A-operand read touches (one 256-byte LDS
  // pass) land on 16 distinct bank groups
  auto dswz = [](int h) { return (h & 7) ^ ((h >> 3) & 1); };
  const int kw0 = key0 + wave * WKEYS;
  const int kw1 = min(n, kw0 + WKEYS);
  // loads are clamped to the wave's own last key (or the block's first key for a wave past the
  // row): the prefetch issued by its last step then re-reads cached lines instead of fetching
  // the next wave's keys
  const int klast = max(kw1 - 1, key0);
  // The contraction runs over the 128 dims in a permuted order, the same for both operands: lane
  // group g takes dims [16g, 16g + 16) and [64 + 16g, 80 + 16g).  A load instruction then reads 64
  // contiguous bytes of each of its 16 keys (the first half of every row, then the second).
  auto load = [&](i32x8 (&dst)[NT], int kb) {
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      const int key = min(kb + 16 * jt + r, klast);
      const uint8_t* p = k_cache + ((int64_t)b * cap + key) * ROWB + g * 16;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 64);
      dst[jt] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // sv[s][jt]: the score of key kw0 + 32 s + 16 jt + r (every lane group holds it after the sum)
  float sv[2][NT] = {};
  auto step = [&](const i32x8 (&bfr)[NT], i32x8 (&nxt)[NT], int kb, float (&out)[NT], bool prefetch) {
    if (prefetch) load(nxt, kb + NT * 16);
    float acc[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) acc[jt] = 0.f;
    for (int hb = 0; hb < H; hb += 16) {
      const uint8_t* qa = q_lds + (hb + r) * ROWB;
      const int hr = dswz(hb + r);
      const i32x4 lo = *reinterpret_cast<const i32x4*>(qa + ((g ^ hr) * 16));
      const i32x4 hi = *reinterpret_cast<const i32x4*>(qa + (((g + 4) ^ hr) * 16));
      const i32x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const f32x4 wv = *reinterpret_cast<const f32x4*>(w_lds + hb + 4 * g);
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        f32x4 c = mfma_fp8_16x16x128(a8, bfr[jt], (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[jt] = fmaf(wv[i], fmaxf(c[i], 0.f), acc[jt]);
      }
    }
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      float v = acc[jt];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      out[jt] = v;
    }
  };
  // all of the wave's keys, the queries and the head weights are requested before any is used:
  // one round trip (a load-then-store loop would wait for each of its loads in turn)
  i32x8 bA[NT], bB[NT];
  load(bA, kw0);
  load(bB, kw0 + NT * 16);
  constexpr int QPT = HMAX * UNITS / 256;  // 16-byte query pieces per thread
  i32x4 qv[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int u = tid + 256 * j, h = u / UNITS, c = u - h * UNITS;
    if (h < H) qv[j] = *reinterpret_cast<const i32x4*>(q_idx + ((int64_t)b * H + h) * ROWB + c * 16);
  }
  const float wv_in = tid < H ? w_idx[(int64_t)b * H + tid] : 0.f;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int u = tid + 256 * j, h = u / UNITS, c = u - h * UNITS;
    if (h < H) *reinterpret_cast<i32x4*>(q_lds + h * ROWB + ((c ^ dswz(h)) * 16)) = qv[j];
  }
  if (tid < H) w_lds[tid] = wv_in;
  __syncthreads();
  if (kw0 < kw1) {
    step(bA, bB, kw0, sv[0], false);
    if (kw0 + NT * 16 < kw1) step(bB, bA, kw0 + NT * 16, sv[1], false);
  }
  // epilogue, one key per lane: lane (r, g) owns key kw0 + 32 (g >> 1) + 16 (g & 1) + r (every
  // lane group holds every score of the wave after the sums)
  const int kidx = 32 * (g >> 1) + 16 * (g & 1) + r;
  const bool kval = kw0 + kidx < kw1;
  const float myv = g == 0 ? sv[0][0] : g == 1 ? sv[0][1] : g == 2 ? sv[1][0] : sv[1][1];
  const uint32_t mykey = score_key(myv);
  // the block's largest order key sets its histogram window
  uint32_t kmax = kval ? mykey : 0u;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  if (lane == 0) red_lds[wave] = kmax;
  lds_sync();
  kmax = max(max(red_lds[0], red_lds[1]), max(red_lds[2], red_lds[3]));
  const int base = decode_win_base(kmax);
  // histogram window; the atomic's return value is the key's rank inside its bin
  const int ib = int(mykey >> kDecodeBinShift) - base;
  const int wbin = ib >= 0 ? ib : kDecodeWinBins;
  const int rank = kval ? atomicAdd(&win_lds[wbin], 1) : 0;
  lds_sync();
  const int64_t slot = (int64_t)b * blk_stride + blockIdx.x;
  if (wave == 0) {
    // bins in descending order: the inclusive count is the window's cumulative count (keys of
    // this bin or higher, written), the exclusive one the bin's first slot; the keys below the
    // window follow the window's keys
    const int c = lane < kDecodeWinBins ? win_lds[kDecodeWinBins - 1 - lane] : 0;
    const int incl = wave_incl_scan(c);
    if (lane < kDecodeWinBins) {
      off_lds[kDecodeWinBins - 1 - lane] = incl - c;
      wcnt[slot * kDecodeWinBins + kDecodeWinBins - 1 - lane] = uint16_t(incl);
    }
    if (lane == 63) off_lds[kDecodeWinBins] = incl;
  }
  lds_sync();
  if (kval) {
    const int d = off_lds[wbin] + rank;
    skeys[slot * kDecodeKeysPerBlock + d] = mykey;
    spos[slot * kDecodeKeysPerBlock + d] = uint8_t(wave * WKEYS + kidx);
  }
  if (tid == 0) wbase[slot] = base;
}

// ------------------------------------------------------------------------------------------
// host-side launchers
// ------------------------------------------------------------------------------------------
hipError_t launch_build_schedule(const int32_t* cu, int nseq, int bq, int nb_bound, int2* sched,
                                 int* count, int64_t* seqoff, hipStream_t st) {
  const int threads = 256;
  const int work = max(nb_bound, nseq + 1);
  build_schedule_kernel<<<(work + threads - 1) / threads, threads, 0, st>>>(cu, nseq, bq, nb_bound,
                                                                            sched, count, seqoff);
  return hipGetLastError();
}

// Triangle mode (seqoff != nullptr): every schedule entry, grid nb_bound, scores at seqoff[b] +
// score_block_offset(j).  Chunk mode (seqoff == nullptr): positions n0 .. n0 + nblocks - 1 of the
// chunked loop (chunk_entry), position n0 + c into slot c (slot_stride floats apart) of the
// buffer `scores`.
hipError_t launch_indexer_prefill(bool fp8, int di, const void* q_idx, const void* k_idx,
                                  const float* w, const int32_t* cu, int H, const int2* sched,
                                  const int* count, int n0, int nblocks, const int64_t* seqoff,
                                  int64_t slot_stride, float* scores, float2* rowrange, hipStream_t st) {
  const auto* q = static_cast<const uint8_t*>(q_idx);
  const auto* k = static_cast<const uint8_t*>(k_idx);
  if (nblocks <= 0) return hipSuccess;
  if (fp8 && di == 128)
    indexer_prefill_kernel<true, 128, 64, 8, 4><<<nblocks, 512, 0, st>>>(q, k, w, cu, H, sched, count, n0, seqoff,
                                                                        slot_stride, scores, rowrange);
  else if (!fp8 && di == 64)
    indexer_prefill_kernel<false, 64, 64, 8, 4><<<nblocks, 512, 0, st>>>(q, k, w, cu, H, sched, count, n0, seqoff,
                                                                        slot_stride, scores, rowrange);
  else if (!fp8 && di == 128)
    indexer_prefill_kernel<false, 128, 32, 8, 1><<<nblocks, 512, 0, st>>>(q, k, w, cu, H, sched, count, n0, seqoff,
                                                                         slot_stride, scores, rowrange);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_unpack_scores(const float* buf, int64_t slot_stride, const int2* sched, const int* count, int n0,
                                int nblocks, const int32_t* cu, int ldo, float* out, hipStream_t st) {
  if (nblocks <= 0) return hipSuccess;
  unpack_scores_kernel<<<(unsigned)nblocks * 16, 256, 0, st>>>(buf, slot_stride, sched, count, n0, cu, ldo, out);
  return hipGetLastError();
}

hipError_t launch_indexer_decode(const void* q_idx, const float* w, const void* k_cache,
                                 const int32_t* cache_lens, int B, int cap, int max_len, int H, uint32_t* skeys,
                                 uint8_t* spos, int* wbase, uint16_t* wcnt, hipStream_t st) {
  dim3 grid((max_len + kDecodeKeysPerBlock - 1) / kDecodeKeysPerBlock, B);
  indexer_decode_kernel<64, 2><<<grid, 256, 0, st>>>(static_cast<const uint8_t*>(q_idx), w,
                                                     static_cast<const uint8_t*>(k_cache), cache_lens,
                                                     cap, H, skeys, spos, wbase, wcnt, (int)grid.x);
  return hipGetLastError();
}

}  // namespace dsa
