// C-ABI host layer of the DSA hot path: argument checks, workspace layout, launch order.
// Every entry point validates on the host, then only enqueues kernels on the caller's stream.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/dsa.h"
#include "common.h"

namespace dsa {
hipError_t launch_build_schedule(const int32_t* cu, int nseq, int bq, int nb_bound, int2* sched, int* count,
                                 int64_t* seqoff, hipStream_t st);
hipError_t launch_indexer_prefill(bool fp8, int di, const void* q_idx, const void* k_idx, const float* w,
                                  const int32_t* cu, int H, const int2* sched, const int* count, int n0, int nblocks,
                                  const int64_t* seqoff, int64_t slot_stride, float* scores, float2* rowrange,
                                  hipStream_t st);
hipError_t launch_unpack_scores(const float* buf, int64_t slot_stride, const int2* sched, const int* count, int n0,
                                int nblocks, const int32_t* cu, int ldo, float* out, hipStream_t st);
hipError_t launch_indexer_decode(const void* q_idx, const float* w, const void* k_cache, const int32_t* cache_lens,
                                 int B, int cap, int max_len, int H, uint32_t* skeys, uint8_t* spos, int* wbase,
                                 uint16_t* wcnt, hipStream_t st);
hipError_t launch_topk_prefill(const float* buf, int64_t slot_stride, const int2* sched, const int* count, int n0,
                               int nblocks, const int32_t* cu, int K, const float2* rowrange, int32_t* out,
                               hipStream_t st);
hipError_t launch_topk_decode(const uint32_t* skeys, const uint8_t* spos, const int32_t* cache_lens, int B,
                              int max_len, int K, const int* wbase, const uint16_t* wcnt, int blk_stride,
                              int32_t* out, hipStream_t st);
hipError_t launch_gather_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx, int K,
                                   int mode, const int32_t* cu, int nseq, const int32_t* cache_lens, int cap,
                                   int64_t rows, int Hq, int Hkv, float scale, int keys_per_split, int nsplit,
                                   uint16_t* out, float* o_part, float2* ml_part, hipStream_t st,
                                   float* lse_out = nullptr, const int32_t* order = nullptr);
int64_t row_order_count_ints(int64_t T, int max_seqlen, int nseq);
hipError_t launch_row_order(const int32_t* idx, int K, const int32_t* cu, int nseq, int64_t T, int max_seqlen,
                            int* sig, int* cnt, int32_t* order, hipStream_t st);
hipError_t launch_union(const int32_t* idx, int K, const int32_t* cu, const int2* sched, const int* count,
                        int nb_bound, int64_t ustride, int32_t* ukeys, uint16_t* umask, int* ucount, hipStream_t st);
hipError_t launch_dedup_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vh, const int32_t* cu, int Hq,
                                  int Hkv, float scale, const int2* sched, const int* count, int nb_bound,
                                  int64_t ustride, const int32_t* ukeys, const uint16_t* umask, const int* ucount,
                                  uint16_t* out, int max_len, hipStream_t st);
hipError_t launch_kl_lse(const uint16_t* q, const uint16_t* k, const int32_t* cu, int Hq, int Hkv, float scale,
                         const int2* sched128, const int* count128, int nb128, float* lse, hipStream_t st);
hipError_t launch_kl_target(const uint16_t* q, const uint16_t* k, const int32_t* cu, int Hq, int Hkv, float scale,
                            const int2* sched128, const int* count128, int nb128, int max_len, const float* lse,
                            const int64_t* seqoff, float* P, hipStream_t st);
hipError_t launch_kl_rows(const float* I, float* P, const int64_t* seqoff, const int32_t* cu, int nseq, int64_t T,
                          const float2* rowrange, float* kl, hipStream_t st);
hipError_t launch_kl_dq(int H, const uint8_t* q_idx, const uint8_t* k_idx, const float* w, const float* G,
                        const int64_t* seqoff, const int32_t* cu, const int2* schedR, const int* countR, int nbR,
                        float* dq, float* dw, hipStream_t st);
int kl_dk_slices(int max_len);
hipError_t launch_kl_dk(int H, const uint8_t* q_idx, const uint8_t* k_idx, const float* w, const float* G,
                        const int64_t* seqoff, const int32_t* cu, int nseq, const int2* sched256,
                        const int* count256, int nb256, int max_len, int64_t T, float* dk_part,
                        float* dk, hipStream_t st);
int bwd_slices(int max_len);
hipError_t launch_bwd_delta(const uint16_t* dout, const uint16_t* out, int64_t pairs, float* D, hipStream_t st);
hipError_t launch_sel_bitmap(const int32_t* idx, int K, const int32_t* cu, const int2* sched32, const int* count32,
                             int nb32, uint32_t* W, hipStream_t st);
hipError_t launch_dedup_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                           const float* lse, const float* Dlt, const int32_t* cu, int Hq, int Hkv, float scale,
                           const int2* sched16, const int* count16, int nb16, int64_t ustride, const int32_t* ukeys,
                           const uint16_t* umask, const int* ucount, float* dq, int max_len, hipStream_t st);
hipError_t launch_to_f16(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t st);
hipError_t launch_bwd_prep(const uint16_t* q, const uint16_t* dout, const float* lse, const float* Dlt,
                           const int32_t* cu, int nseq, int64_t T, int Hq, int Hkv, uint16_t* qh, uint16_t* doh,
                           uint16_t* qt, uint16_t* dot, float* stats, hipStream_t st);
int64_t bwd_cols(int64_t T, int G, int nseq);
hipError_t launch_sparse_dkv(const uint16_t* qh, const uint16_t* kh, const uint16_t* vh, const uint16_t* doh,
                             const uint16_t* qt, const uint16_t* dot, const float* stats, const int32_t* cu, int nseq,
                             int Hq, int Hkv, float scale, const int2* sched128, const int* count128, int nb128,
                             const uint32_t* W, int max_len, int64_t T, float* dk_part, float* dv_part, float* dk,
                             float* dv, hipStream_t st);
hipError_t launch_topk_general(const float* scores, int64_t rows, int n, int64_t ld, const int32_t* lens, int K,
                               int32_t* out, hipStream_t st);
int64_t dense_vt_cols(int64_t T, int nseq);
hipError_t launch_dense_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* vt, int64_t T,
                                const int32_t* cu, int nseq, int Hq, int Hkv, float scale, const int2* sched,
                                const int* count, int nb_bound, uint16_t* out, hipStream_t st);

// Copy one new token per sequence into the caches at row lens[b] and count it (lens[b] += 1);
// a full cache (lens[b] >= cap) is left untouched.  Rows are moved in 16-byte units (VEC) when
// every row size and base pointer allows it, else byte by byte.
template <bool VEC>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint8_t* __restrict__ kin,
                                                        const uint8_t* __restrict__ knew,
                                                        const uint8_t* __restrict__ vnew, int32_t* __restrict__ lens,
                                                        int cap, int idx_row_bytes, int kv_row_bytes,
                                                        uint8_t* __restrict__ kic, uint8_t* __restrict__ kc,
                                                        uint8_t* __restrict__ vc) {
  const int b = blockIdx.x;
  const int pos = lens[b];
  if (pos < 0 || pos >= cap) return;
  const int64_t row = (int64_t)b * cap + pos;
  const int U = VEC ? 16 : 1;
  const int ni = idx_row_bytes / U, nk = kv_row_bytes / U;
  for (int i = threadIdx.x; i < ni + 2 * nk; i += blockDim.x) {
    const uint8_t* src;
    uint8_t* dst;
    if (i < ni) {
      src = kin + ((int64_t)b * ni + i) * U;
      dst = kic + (row * ni + i) * U;
    } else if (i < ni + nk) {
      src = knew + ((int64_t)b * nk + i - ni) * U;
      dst = kc + (row * nk + i - ni) * U;
    } else {
      src = vnew + ((int64_t)b * nk + i - ni - nk) * U;
      dst = vc + (row * nk + i - ni - nk) * U;
    }
    if (VEC) *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    else *dst = *src;
  }
  __syncthreads();  // every thread has read lens[b] before it changes
  if (threadIdx.x == 0) lens[b] = pos + 1;
}
}  // namespace dsa

using namespace dsa;

// Device memory of the allocation-free decode entry point: a file-scope array that each GPU the
// library runs on holds from module load until the process ends.  In host code its name is only
// a stand-in; the per-device address comes from hipGetSymbolAddress and is kept below.
constexpr size_t kDecodeScratchBytes = size_t(DSA_DECODE_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return DSA_OK;
  g_last_hip_error = int(e);
  return DSA_ERR_HIP;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_heads(int32_t topk, int32_t H, int32_t dI, int32_t dtype, int32_t Hq, int32_t Hkv, int32_t d,
                float scale, bool need_indexer) {
  if (topk < 1 || topk > 4096) return DSA_ERR_INVALID_ARGUMENT;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return DSA_ERR_INVALID_ARGUMENT;
  if (!(scale > 0.f) || !isfinite(scale)) return DSA_ERR_INVALID_ARGUMENT;
  if (Hkv > 8 || Hq / Hkv > 16) return DSA_ERR_UNSUPPORTED;
  if (d != 128) return DSA_ERR_UNSUPPORTED;
  if (need_indexer) {
    if (H < 1 || dI < 1) return DSA_ERR_INVALID_ARGUMENT;
    if (dtype != DSA_IDX_BF16 && dtype != DSA_IDX_FP8_E4M3) return DSA_ERR_INVALID_ARGUMENT;
    if (H % 16 != 0 || H > 64) return DSA_ERR_UNSUPPORTED;
    if (dtype == DSA_IDX_FP8_E4M3 && dI != 128) return DSA_ERR_UNSUPPORTED;
    if (dtype == DSA_IDX_BF16 && dI != 64 && dI != 128) return DSA_ERR_UNSUPPORTED;
    if (dtype == DSA_IDX_BF16 && dI == 128 && H > 32) return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

// K/V rows are addressed with 32-bit byte offsets from a sequence's (or a cache's) first row:
// rows x Hkv x head_dim x 2 bytes must stay below 4 GiB.
bool kv_span_fits(int64_t rows, int kv_heads, int head_dim) {
  return uint64_t(rows) * uint64_t(kv_heads) * uint64_t(head_dim) * 2 <= 0xFFFFFFFFull;
}

// uses_kv: the entry point runs attention kernels (everything but the index-only calls)
int check_prefill(const dsa_prefill_shape* s, bool need_indexer, bool uses_kv = true) {
  if (!s || !s->cu_seqlens || s->num_seqs < 1 || s->total_tokens < 0 || s->max_seqlen < 0)
    return DSA_ERR_INVALID_ARGUMENT;
  if (s->total_tokens > 0 && s->max_seqlen < 1) return DSA_ERR_INVALID_ARGUMENT;
  if (s->max_seqlen > s->total_tokens) return DSA_ERR_INVALID_ARGUMENT;
  if (s->total_tokens > (int64_t(1) << 31) - 1) return DSA_ERR_UNSUPPORTED;
  const int rc = check_heads(s->topk, s->idx_heads, s->idx_dim, s->idx_dtype, s->q_heads, s->kv_heads, s->head_dim,
                             s->softmax_scale, need_indexer);
  if (rc) return rc;
  if (uses_kv && !kv_span_fits(s->total_tokens, s->kv_heads, s->head_dim)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

// Prefill workspace layout (all offsets 256-byte aligned):
//   counts int[64] | seqoff int64[B+1] | sched16 int2[nb16] | sched128 int2[nb128] |
//   rowrange float2[T] | chunk buffer float[kChunkBlocks][slot_stride] | topk int32[T*k] |
//   row order (signatures, counts, order) | V in fp16 (dense reference only)
// The indexer scores its 16-row blocks in chunks of kChunkBlocks blocks, one block per slot of
// the chunk buffer, in the order chunk_entry gives (each chunk: the next kPairHalf longest blocks
// of the longest-first schedule, then kPairHalf from its short end, so a compute unit that
// finishes a long block early takes the longest short one); the top-k then selects the chunk's
// rows before the next chunk reuses the buffer.  A slot holds a block of the longest rows (16
// rows of max_seqlen rounded up to 16 scores), so the buffer is kChunkBlocks x 16 x max_seqlen
// floats (4 GiB at 131072 tokens) whatever the batch holds.
constexpr int kChunkBlocks = 2 * kPairHalf;  // the long and the short half of a chunk (chunk_entry)

struct PrefillWs {
  size_t counts, seqoff, sched16, sched128, rowrange, scores, topk, osig, ocnt, order, v16, total;
  int nb16, nb128, nchunks;
  int64_t slot_stride, score_floats;
};

// Floats of the whole score triangle (16-row blocks, block j of 16(j+1) scores per row): exact
// from host lengths, else the bound for T tokens in sequences of at most max_seqlen.
int64_t triangle_floats(const dsa_prefill_shape* s, const int32_t* cu_host) {
  int64_t sq = 0;
  if (cu_host) {
    for (int b = 0; b < s->num_seqs; ++b) {
      const int64_t n16 = (int64_t(cu_host[b + 1]) - cu_host[b] + 15) / 16;
      sq += n16 * (n16 + 1);
    }
  } else {
    const int64_t nb16 = (s->total_tokens + 15) / 16 + s->num_seqs;
    const int64_t M = (int64_t(s->max_seqlen) + 15) / 16;
    if (M > 0) {
      const int64_t q = nb16 / M, rem = nb16 % M;
      sq = q * M * (M + 1) + rem * (rem + 1);
    }
  }
  return 128 * sq;
}

PrefillWs prefill_layout(const dsa_prefill_shape* s, const int32_t* cu_host) {
  PrefillWs w{};
  const int64_t T = s->total_tokens;
  const int B = s->num_seqs;
  int64_t nb16 = 0, nb128 = 0;
  if (cu_host) {
    for (int b = 0; b < B; ++b) {
      const int64_t L = cu_host[b + 1] - cu_host[b];
      nb16 += (L + 15) / 16;
      nb128 += (L + 127) / 128;
    }
  } else {
    nb16 = (T + 15) / 16 + B;
    nb128 = (T + 127) / 128 + B;
  }
  w.nb16 = int(nb16);
  w.nb128 = int(nb128);
  w.nchunks = int((nb16 + kChunkBlocks - 1) / kChunkBlocks);
  w.slot_stride = 16 * ((int64_t(s->max_seqlen) + 15) / 16 * 16);
  w.score_floats = int64_t(kChunkBlocks) * w.slot_stride;
  size_t off = 0;
  w.counts = off; off = align_up(off + 64 * sizeof(int), 256);
  w.seqoff = off; off = align_up(off + size_t(B + 1) * sizeof(int64_t), 256);
  w.sched16 = off; off = align_up(off + size_t(nb16) * sizeof(int2), 256);
  w.sched128 = off; off = align_up(off + size_t(nb128) * sizeof(int2), 256);
  w.rowrange = off; off = align_up(off + size_t(T) * sizeof(float2), 256);
  w.scores = off; off = align_up(off + size_t(w.score_floats) * sizeof(float), 256);
  w.topk = off; off = align_up(off + size_t(T) * size_t(s->topk) * sizeof(int32_t), 256);
  // gather row order: per-row key, per-key counts / offsets, the order itself
  w.osig = off; off = align_up(off + size_t(T) * sizeof(int), 256);
  w.ocnt = off; off = align_up(off + size_t(row_order_count_ints(T, s->max_seqlen, B)) * sizeof(int), 256);
  w.order = off; off = align_up(off + size_t(T) * sizeof(int32_t), 256);
  // V^T in fp16 for the dense reference (dense_causal_attention only), 64 zero columns after
  // each sequence
  w.v16 = off;
  off = align_up(off + size_t(dense_vt_cols(T, B)) * size_t(s->kv_heads) * size_t(s->head_dim) * sizeof(uint16_t), 256);
  w.total = off;
  return w;
}

template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

// Indexer scores of chunk c (loop positions c * kChunkBlocks .., chunk_entry) into the chunk buffer.
hipError_t index_chunk(const dsa_prefill_shape* s, const void* q_idx, const void* k_idx, const float* w_idx,
                       void* ws, const PrefillWs& L, int c, hipStream_t st) {
  return launch_indexer_prefill(s->idx_dtype == DSA_IDX_FP8_E4M3, s->idx_dim, q_idx, k_idx, w_idx, s->cu_seqlens,
                                s->idx_heads, at<int2>(ws, L.sched16), at<int>(ws, L.counts), c * kChunkBlocks,
                                kChunkBlocks, nullptr, L.slot_stride, at<float>(ws, L.scores),
                                at<float2>(ws, L.rowrange), st);
}

hipError_t topk_chunk(const dsa_prefill_shape* s, void* ws, const PrefillWs& L, int c, int32_t* idx, hipStream_t st) {
  return launch_topk_prefill(at<float>(ws, L.scores), L.slot_stride, at<int2>(ws, L.sched16), at<int>(ws, L.counts),
                             c * kChunkBlocks, kChunkBlocks, s->cu_seqlens, s->topk, at<float2>(ws, L.rowrange), idx,
                             st);
}

hipError_t build_schedule16(const dsa_prefill_shape* s, void* ws, const PrefillWs& L, hipStream_t st) {
  return launch_build_schedule(s->cu_seqlens, s->num_seqs, 16, L.nb16, at<int2>(ws, L.sched16), at<int>(ws, L.counts),
                               at<int64_t>(ws, L.seqoff), st);
}

// Dedup workspace layout (adjacent-query union per 16-row block; 256-byte aligned):
//   counts int[64] | sched16 int2[nb16] | ucount int[nb16] | ukeys int32[nb16][16k] | umask uint16[nb16][16k] |
//   fp16 copy of V [T][Hkv][128]
struct DedupWs {
  size_t counts, sched16, ucount, ukeys, umask, vh, total;
  int nb16;
  int64_t ustride;
};

DedupWs dedup_layout(const dsa_prefill_shape* s) {
  DedupWs w{};
  w.nb16 = int((s->total_tokens + 15) / 16 + s->num_seqs);
  w.ustride = 16 * int64_t(s->topk);
  size_t off = 0;
  w.counts = off; off = align_up(off + 64 * sizeof(int), 256);
  w.sched16 = off; off = align_up(off + size_t(w.nb16) * sizeof(int2), 256);
  w.ucount = off; off = align_up(off + size_t(w.nb16) * sizeof(int), 256);
  w.ukeys = off; off = align_up(off + size_t(w.nb16) * size_t(w.ustride) * sizeof(int32_t), 256);
  w.umask = off; off = align_up(off + size_t(w.nb16) * size_t(w.ustride) * sizeof(uint16_t), 256);
  w.vh = off; off = align_up(off + size_t(s->total_tokens) * size_t(s->kv_heads) * 128 * sizeof(uint16_t), 256);
  w.total = off;
  return w;
}

// Warm-up KL workspace: the prefill layout (schedules, row ranges, indexer score triangle) then
//   P triangle float[score_floats] | lse float[T][Hq] | schedR int2[nbR] | sched256 int2[nb256] |
//   dk partials float[slices][T][128].  counts[2] / counts[3] hold the R-row / 256-row schedule
//   sizes.
struct KlWs {
  PrefillWs base;
  size_t tri, P, lse, schedR, sched256, dkpart, total;
  int R, nbR, nb256, slices;
  int64_t tri_floats;
};

KlWs kl_layout(const dsa_prefill_shape* s) {
  KlWs w{};
  w.base = prefill_layout(s, nullptr);
  const int64_t T = s->total_tokens;
  w.R = 256 / (s->idx_heads > 0 ? s->idx_heads : 1);
  w.nbR = int((T + w.R - 1) / w.R + s->num_seqs);
  w.nb256 = int((T + 255) / 256 + s->num_seqs);
  w.slices = kl_dk_slices(s->max_seqlen);
  // the objective covers every causal pair: the indexer scores and the target distribution are
  // both whole score triangles
  w.tri_floats = triangle_floats(s, nullptr);
  size_t off = w.base.total;
  w.tri = off; off = align_up(off + size_t(w.tri_floats) * sizeof(float), 256);
  w.P = off; off = align_up(off + size_t(w.tri_floats) * sizeof(float), 256);
  w.lse = off; off = align_up(off + size_t(T) * size_t(s->q_heads) * sizeof(float), 256);
  w.schedR = off; off = align_up(off + size_t(w.nbR) * sizeof(int2), 256);
  w.sched256 = off; off = align_up(off + size_t(w.nb256) * sizeof(int2), 256);
  w.dkpart = off; off = align_up(off + size_t(w.slices) * size_t(T) * 128 * sizeof(float), 256);
  w.total = off;
  return w;
}

int check_kl(const dsa_prefill_shape* s) {
  int rc = check_prefill(s, true);
  if (rc) return rc;
  if (s->idx_dtype != DSA_IDX_FP8_E4M3 || s->idx_dim != 128) return DSA_ERR_UNSUPPORTED;
  if (s->idx_heads != 16 && s->idx_heads != 32 && s->idx_heads != 64) return DSA_ERR_UNSUPPORTED;
  if (s->kv_heads != 1 && s->kv_heads != 2 && s->kv_heads != 4) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

// Sparse attention backward workspace: counts int[64] (0: 16-row, 1: 32-row, 2: 128-key
// schedule sizes) | D float[T][Hq] | sched16 | sched32 | sched128 | ucount int[nb16] |
// ukeys int32[nb16][16k] | umask uint16[nb16][16k] | bitmap uint32[(max_len/32 + 1)(T + 3B) + 128] |
// dk, dv partials float[slices][T][Hkv][128] each | fp16 q, k, v, dO | transposed fp16 q, dO
// [Hkv][128][cols] | statistics float[Hkv][2][cols] (cols = bwd_cols(T, G, B)).
struct BwdWs {
  size_t counts, delta, sched16, sched32, sched128, ucount, ukeys, umask, bitmap, dkpart, dvpart, qh, kh, vh, doh,
      qt, dot, stats, total;
  int nb16, nb32, nb128;
  int64_t ustride;
};

BwdWs bwd_layout(const dsa_prefill_shape* s) {
  BwdWs w{};
  const int64_t T = s->total_tokens;
  const int B = s->num_seqs;
  w.nb16 = int((T + 15) / 16 + B);
  w.nb32 = int((T + 31) / 32 + B);
  w.nb128 = int((T + 127) / 128 + B);
  w.ustride = 16 * int64_t(s->topk);
  const size_t parts = size_t(bwd_slices(s->max_seqlen)) * size_t(T) * size_t(s->kv_heads) * 128 * sizeof(float);
  size_t off = 0;
  w.counts = off; off = align_up(off + 64 * sizeof(int), 256);
  w.delta = off; off = align_up(off + size_t(T) * size_t(s->q_heads) * sizeof(float), 256);
  w.sched16 = off; off = align_up(off + size_t(w.nb16) * sizeof(int2), 256);
  w.sched32 = off; off = align_up(off + size_t(w.nb32) * sizeof(int2), 256);
  w.sched128 = off; off = align_up(off + size_t(w.nb128) * sizeof(int2), 256);
  w.ucount = off; off = align_up(off + size_t(w.nb16) * sizeof(int), 256);
  w.ukeys = off; off = align_up(off + size_t(w.nb16) * size_t(w.ustride) * sizeof(int32_t), 256);
  w.umask = off; off = align_up(off + size_t(w.nb16) * size_t(w.ustride) * sizeof(uint16_t), 256);
  w.bitmap = off;
  off = align_up(off + (size_t(s->max_seqlen / 32 + 1) * size_t(T + 3 * B) + 128) * sizeof(uint32_t), 256);
  w.dkpart = off; off = align_up(off + parts, 256);
  w.dvpart = off; off = align_up(off + parts, 256);
  // fp16 copies of Q, K, V and dO for the gradient products
  w.qh = off; off = align_up(off + size_t(T) * size_t(s->q_heads) * 128 * sizeof(uint16_t), 256);
  w.kh = off; off = align_up(off + size_t(T) * size_t(s->kv_heads) * 128 * sizeof(uint16_t), 256);
  w.vh = off; off = align_up(off + size_t(T) * size_t(s->kv_heads) * 128 * sizeof(uint16_t), 256);
  w.doh = off; off = align_up(off + size_t(T) * size_t(s->q_heads) * 128 * sizeof(uint16_t), 256);
  const size_t cols = size_t(bwd_cols(T, s->q_heads / s->kv_heads, B));
  w.qt = off; off = align_up(off + size_t(s->kv_heads) * 128 * cols * sizeof(uint16_t), 256);
  w.dot = off; off = align_up(off + size_t(s->kv_heads) * 128 * cols * sizeof(uint16_t), 256);
  w.stats = off; off = align_up(off + size_t(s->kv_heads) * 2 * cols * sizeof(float), 256);
  w.total = off;
  return w;
}

bool dedup_supported(const dsa_prefill_shape* s) {
  const int G = s->q_heads / s->kv_heads;
  return G == 2 || G == 4 || G == 8 || G == 16;
}

int check_prefill_ws(const dsa_prefill_shape* s, void* ws, size_t ws_bytes, PrefillWs* L) {
  *L = prefill_layout(s, nullptr);
  if (!ws || !aligned16(ws)) return DSA_ERR_INVALID_ARGUMENT;
  // the exact layout (from device cu_seqlens) never exceeds the host bound
  if (ws_bytes < L->total) return DSA_ERR_WORKSPACE_TOO_SMALL;
  return DSA_OK;
}

constexpr int kDecodeMaxCacheLen = 1 << 20;  // longest decode cache (rows)

int check_decode(const dsa_decode_shape* s, bool need_indexer) {
  if (!s || !s->cache_lens || s->batch < 1 || s->cache_capacity < 1) return DSA_ERR_INVALID_ARGUMENT;
  if (s->max_cache_len < 1 || s->max_cache_len > s->cache_capacity) return DSA_ERR_INVALID_ARGUMENT;
  if (s->max_cache_len > kDecodeMaxCacheLen) return DSA_ERR_UNSUPPORTED;
  int rc = check_heads(s->topk, s->idx_heads, s->idx_dim, s->idx_dtype, s->q_heads, s->kv_heads, s->head_dim,
                       s->softmax_scale, need_indexer);
  if (rc) return rc;
  if (need_indexer && s->idx_dtype != DSA_IDX_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
  if (!kv_span_fits(s->cache_capacity, s->kv_heads, s->head_dim)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

constexpr int kDecodeSparseSplit = 128;   // selected keys per split (decode)
constexpr int kDecodeDenseSplit = 2048;   // cache rows per split (dense decode)

struct DecodeWs {
  size_t skeys, spos, topk, opart, mlpart, wbase, wcnt, total;
  int nsplit_sparse, nsplit_dense, blk_stride;
};

// Decode workspace layout (256-byte aligned), per indexer block of kDecodeKeysPerBlock cache rows:
// bin-sorted order keys uint32 [B][blk][256] and their block positions uint8 [B][blk][256] |
// topk int32 [B][k] | split partials (sized for the larger of the sparse and dense split counts) |
// histogram window base int [B][blk] and counts uint16 [B][blk][kDecodeWinBins].
// Every byte the decode kernels read is written earlier in the same call.
DecodeWs decode_layout(const dsa_decode_shape* s) {
  DecodeWs w{};
  w.nsplit_sparse = (s->topk + kDecodeSparseSplit - 1) / kDecodeSparseSplit;
  w.nsplit_dense = (s->max_cache_len + kDecodeDenseSplit - 1) / kDecodeDenseSplit;
  w.blk_stride = (s->max_cache_len + kDecodeKeysPerBlock - 1) / kDecodeKeysPerBlock;
  const int ns = w.nsplit_sparse > w.nsplit_dense ? w.nsplit_sparse : w.nsplit_dense;
  const size_t B = size_t(s->batch);
  size_t off = 0;
  const size_t slots = B * size_t(w.blk_stride) * kDecodeKeysPerBlock;
  w.skeys = off; off = align_up(off + slots * sizeof(uint32_t), 256);
  w.spos = off; off = align_up(off + slots, 256);
  w.topk = off; off = align_up(off + B * size_t(s->topk) * sizeof(int32_t), 256);
  w.opart = off; off = align_up(off + B * ns * size_t(s->q_heads) * s->head_dim * sizeof(float), 256);
  w.mlpart = off; off = align_up(off + B * ns * size_t(s->q_heads) * sizeof(float2), 256);
  w.wbase = off; off = align_up(off + B * size_t(w.blk_stride) * sizeof(int), 256);
  w.wcnt = off; off = align_up(off + B * size_t(w.blk_stride) * kDecodeWinBins * sizeof(uint16_t), 256);
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DSA_ERR_HIP: return "HIP launch error";
    case DSA_ERR_SCRATCH_TOO_SMALL: return "shape needs more than the static decode scratch";
    default: return "unknown status";
  }
}

int dsa_last_hip_error(void) { return g_last_hip_error; }

int dsa_prefill_timing_events(const dsa_prefill_shape* s, int32_t* count) {
  if (!count) return DSA_ERR_INVALID_ARGUMENT;
  int rc = check_prefill(s, false, false);
  if (rc) return rc;
  *count = 3 + 2 * prefill_layout(s, nullptr).nchunks;
  return DSA_OK;
}

int dsa_prefill_workspace_size(const dsa_prefill_shape* s, const int32_t* cu_seqlens_host, size_t* bytes) {
  if (!bytes) return DSA_ERR_INVALID_ARGUMENT;
  int rc = check_prefill(s, false, false);
  if (rc) return rc;
  if (s->total_tokens == 0) return DSA_OK;  // empty batch: nothing to do, pointers may be null
  *bytes = prefill_layout(s, cu_seqlens_host).total;
  // the library only checks the host bound, so never report less than it
  const size_t bound = prefill_layout(s, nullptr).total;
  if (*bytes < bound) *bytes = bound;
  return DSA_OK;
}

int dsa_index_scores(const dsa_prefill_shape* s, const void* q_idx, const void* k_idx, const float* w_idx,
                     float* scores, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_prefill(s, true, false);
  if (rc) return rc;
  if (s->total_tokens == 0) return DSA_OK;  // empty batch: nothing to do, pointers may be null
  if (!q_idx || !k_idx || !w_idx || !scores) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx)) return DSA_ERR_INVALID_ARGUMENT;
  PrefillWs L;
  if ((rc = check_prefill_ws(s, ws, ws_bytes, &L))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = build_schedule16(s, ws, L, st);
  for (int c = 0; c < L.nchunks && e == hipSuccess; ++c) {
    e = index_chunk(s, q_idx, k_idx, w_idx, ws, L, c, st);
    if (e == hipSuccess)
      e = launch_unpack_scores(at<float>(ws, L.scores), L.slot_stride, at<int2>(ws, L.sched16), at<int>(ws, L.counts),
                               c * kChunkBlocks, kChunkBlocks, s->cu_seqlens, s->max_seqlen, scores, st);
  }
  return hip_status(e);
}

int dsa_index_topk(const dsa_prefill_shape* s, const void* q_idx, const void* k_idx, const float* w_idx,
                   int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_prefill(s, true, false);
  if (rc) return rc;
  if (s->total_tokens == 0) return DSA_OK;  // empty batch: nothing to do, pointers may be null
  if (!q_idx || !k_idx || !w_idx || !topk_idx) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx)) return DSA_ERR_INVALID_ARGUMENT;
  PrefillWs L;
  if ((rc = check_prefill_ws(s, ws, ws_bytes, &L))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = build_schedule16(s, ws, L, st);
  for (int c = 0; c < L.nchunks && e == hipSuccess; ++c) {
    e = index_chunk(s, q_idx, k_idx, w_idx, ws, L, c, st);
    if (e == hipSuccess) e = topk_chunk(s, ws, L, c, topk_idx, st);
  }
  return hip_status(e);
}

int dsa_sparse_attention(const dsa_prefill_shape* s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* topk_idx, uint16_t* out, void* stream) {
  int rc = check_prefill(s, false);
  if (rc) return rc;
  if (s->total_tokens == 0) return DSA_OK;  // empty batch: nothing to do, pointers may be null
  if (!q || !k || !v || !topk_idx || !out) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return DSA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_gather_attention(q, k, v, topk_idx, s->topk, 0, s->cu_seqlens, s->num_seqs, nullptr, 0,
                                            s->total_tokens, s->q_heads, s->kv_heads, s->softmax_scale, 1 << 30, 1,
                                            out, nullptr, nullptr, static_cast<hipStream_t>(stream)));
}

namespace {
int record(void* const* ev, int i, hipStream_t st) {
  if (!ev) return DSA_OK;
  return hip_status(hipEventRecord(static_cast<hipEvent_t>(ev[i]), st));
}

// Union + masked attention over given indices, with a 16-row block schedule already built.
int dedup_attention(const dsa_prefill_shape* s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int32_t* idx, uint16_t* out, const int2* sched16, const int* count, int nb16,
                    void* dws, const DedupWs& D, hipStream_t st) {
  int rc;
  if ((rc = hip_status(launch_union(idx, s->topk, s->cu_seqlens, sched16, count, nb16, D.ustride,
                                    at<int32_t>(dws, D.ukeys), at<uint16_t>(dws, D.umask), at<int>(dws, D.ucount),
                                    st))))
    return rc;
  uint16_t* vh = at<uint16_t>(dws, D.vh);
  if ((rc = hip_status(launch_to_f16(v, vh, s->total_tokens * s->kv_heads * 128, st)))) return rc;
  return hip_status(launch_dedup_attention(q, k, vh, s->cu_seqlens, s->q_heads, s->kv_heads, s->softmax_scale,
                                           sched16, count, nb16, D.ustride, at<int32_t>(dws, D.ukeys),
                                           at<uint16_t>(dws, D.umask), at<int>(dws, D.ucount), out, s->max_seqlen,
                                           st));
}

int check_dedup_ws(const dsa_prefill_shape* s, void* dws, size_t dws_bytes, DedupWs* D) {
  if (!dedup_supported(s)) return DSA_ERR_UNSUPPORTED;
  *D = dedup_layout(s);
  if (!dws || !aligned16(dws)) return DSA_ERR_INVALID_ARGUMENT;
  if (dws_bytes < D->total) return DSA_ERR_WORKSPACE_TOO_SMALL;
  return DSA_OK;
}

int prefill_impl(const dsa_prefill_shape* s, const void* q_idx, const void* k_idx, const float* w_idx,
                 const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int32_t* topk_idx,
                 void* ws, size_t ws_bytes, void* stream, void* const* ev, void* dws = nullptr,
                 size_t dws_bytes = 0, bool dedup = false) {
  int rc = check_prefill(s, true);
  if (rc) return rc;
  DedupWs D{};
  if (dedup && s->total_tokens > 0 && (rc = check_dedup_ws(s, dws, dws_bytes, &D))) return rc;
  // timing events (dsa_prefill_timed): [0] schedule, then per chunk c [1 + 2c] indexer and
  // [2 + 2c] top-k, then [1 + 2n] row order and [2 + 2n] attention, n = the chunk count
  const int nch = prefill_layout(s, nullptr).nchunks;
  if (s->total_tokens == 0) {  // empty batch: nothing to compute, pointers may be null
    for (int i = 0; i < 3 + 2 * nch && ev; ++i)
      if ((rc = record(ev, i, static_cast<hipStream_t>(stream)))) return rc;
    return DSA_OK;
  }
  if (!q_idx || !k_idx || !w_idx || !q || !k || !v || !out) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx) || !aligned16(q) || !aligned16(k) ||
      !aligned16(v) || !aligned16(out))
    return DSA_ERR_INVALID_ARGUMENT;
  PrefillWs L;
  if ((rc = check_prefill_ws(s, ws, ws_bytes, &L))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.topk);
  hipError_t e = build_schedule16(s, ws, L, st);
  if (e != hipSuccess) return hip_status(e);
  if ((rc = record(ev, 0, st))) return rc;
  for (int c = 0; c < L.nchunks; ++c) {
    if ((rc = hip_status(index_chunk(s, q_idx, k_idx, w_idx, ws, L, c, st)))) return rc;
    if ((rc = record(ev, 1 + 2 * c, st))) return rc;
    if ((rc = hip_status(topk_chunk(s, ws, L, c, idx, st)))) return rc;
    if ((rc = record(ev, 2 + 2 * c, st))) return rc;
  }
  // the gather takes rows in the order of their dominant key block (identity when the key
  // space is too large to sort); this post-processing of the selection counts to the top-k stage
  const int32_t* order = nullptr;
  if (!dedup && row_order_count_ints(s->total_tokens, s->max_seqlen, s->num_seqs) > 0) {
    if ((rc = hip_status(launch_row_order(idx, s->topk, s->cu_seqlens, s->num_seqs, s->total_tokens, s->max_seqlen,
                                          at<int>(ws, L.osig), at<int>(ws, L.ocnt), at<int32_t>(ws, L.order), st))))
      return rc;
    order = at<int32_t>(ws, L.order);
  }
  if ((rc = record(ev, 1 + 2 * nch, st))) return rc;
  if (dedup) {
    if ((rc = dedup_attention(s, q, k, v, idx, out, at<int2>(ws, L.sched16), at<int>(ws, L.counts), L.nb16, dws, D,
                              st)))
      return rc;
  } else {
    if ((rc = hip_status(launch_gather_attention(q, k, v, idx, s->topk, 0, s->cu_seqlens, s->num_seqs, nullptr, 0,
                                                 s->total_tokens, s->q_heads, s->kv_heads, s->softmax_scale, 1 << 30,
                                                 1, out, nullptr, nullptr, st, nullptr, order))))
      return rc;
  }
  return record(ev, 2 + 2 * nch, st);
}

int decode_impl(const dsa_decode_shape* s, const void* q_idx, const float* w_idx, const uint16_t* q,
                const void* k_idx_cache, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* out,
                int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream, void* const* ev) {
  int rc = check_decode(s, true);
  if (rc) return rc;
  if (!q_idx || !w_idx || !q || !k_idx_cache || !k_cache || !v_cache || !out || !ws) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_idx) || !aligned16(w_idx) || !aligned16(q) || !aligned16(k_idx_cache) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out) || !aligned16(ws))
    return DSA_ERR_INVALID_ARGUMENT;
  const DecodeWs L = decode_layout(s);
  if (ws_bytes < L.total) return DSA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.topk);
  uint32_t* skeys = at<uint32_t>(ws, L.skeys);
  uint8_t* spos = at<uint8_t>(ws, L.spos);
  if ((rc = hip_status(launch_indexer_decode(q_idx, w_idx, k_idx_cache, s->cache_lens, s->batch, s->cache_capacity,
                                             s->max_cache_len, s->idx_heads, skeys, spos, at<int>(ws, L.wbase),
                                             at<uint16_t>(ws, L.wcnt), st))))
    return rc;
  if ((rc = record(ev, 0, st))) return rc;
  if ((rc = hip_status(launch_topk_decode(skeys, spos, s->cache_lens, s->batch, s->max_cache_len, s->topk,
                                          at<int>(ws, L.wbase), at<uint16_t>(ws, L.wcnt), L.blk_stride, idx, st))))
    return rc;
  if ((rc = record(ev, 1, st))) return rc;
  if ((rc = hip_status(launch_gather_attention(q, k_cache, v_cache, idx, s->topk, 1, nullptr, 0, s->cache_lens,
                                               s->cache_capacity, s->batch, s->q_heads, s->kv_heads,
                                               s->softmax_scale, kDecodeSparseSplit, L.nsplit_sparse, out,
                                               at<float>(ws, L.opart), at<float2>(ws, L.mlpart), st))))
    return rc;
  return record(ev, 2, st);
}
}  // namespace

int dsa_prefill(const dsa_prefill_shape* s, const void* q_idx, const void* k_idx, const float* w_idx,
                const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int32_t* topk_idx,
                void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl(s, q_idx, k_idx, w_idx, q, k, v, out, topk_idx, ws, ws_bytes, stream, nullptr);
}

int dsa_prefill_timed(const dsa_prefill_shape* s, const void* q_idx, const void* k_idx, const float* w_idx,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int32_t* topk_idx,
                      void* ws, size_t ws_bytes, void* stream, void* const* events) {
  if (!events) return DSA_ERR_INVALID_ARGUMENT;
  return prefill_impl(s, q_idx, k_idx, w_idx, q, k, v, out, topk_idx, ws, ws_bytes, stream, events);
}

int dsa_indexer_kl_workspace_size(const dsa_prefill_shape* s, size_t* bytes) {
  if (!bytes) return DSA_ERR_INVALID_ARGUMENT;
  int rc = check_kl(s);
  if (rc) return rc;
  *bytes = kl_layout(s).total;
  return DSA_OK;
}

int dsa_indexer_kl(const dsa_prefill_shape* s, const void* q_idx, const void* k_idx, const float* w_idx,
                   const uint16_t* q, const uint16_t* k, float* kl, float* dq_idx, float* dk_idx, float* dw_idx,
                   void* ws, size_t ws_bytes, void* stream) {
  int rc = check_kl(s);
  if (rc) return rc;
  if (s->total_tokens == 0) return DSA_OK;
  if (!q_idx || !k_idx || !w_idx || !q || !k || !kl || !dq_idx || !dk_idx || !dw_idx || !ws)
    return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx) || !aligned16(q) || !aligned16(k) ||
      !aligned16(dq_idx) || !aligned16(dk_idx) || !aligned16(ws))
    return DSA_ERR_INVALID_ARGUMENT;
  const KlWs K = kl_layout(s);
  if (ws_bytes < K.total) return DSA_ERR_WORKSPACE_TOO_SMALL;
  const PrefillWs& L = K.base;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int* counts = at<int>(ws, L.counts);
  hipError_t e;
  if ((e = launch_build_schedule(s->cu_seqlens, s->num_seqs, 16, L.nb16, at<int2>(ws, L.sched16), counts,
                                 at<int64_t>(ws, L.seqoff), st)) != hipSuccess ||
      (e = launch_build_schedule(s->cu_seqlens, s->num_seqs, 128, L.nb128, at<int2>(ws, L.sched128), counts + 1,
                                 nullptr, st)) != hipSuccess ||
      (e = launch_build_schedule(s->cu_seqlens, s->num_seqs, K.R, K.nbR, at<int2>(ws, K.schedR), counts + 2, nullptr,
                                 st)) != hipSuccess ||
      (e = launch_build_schedule(s->cu_seqlens, s->num_seqs, 256, K.nb256, at<int2>(ws, K.sched256), counts + 3,
                                 nullptr, st)) != hipSuccess)
    return hip_status(e);
  const int64_t* seqoff = at<int64_t>(ws, L.seqoff);
  float* scores = at<float>(ws, K.tri);
  float* P = at<float>(ws, K.P);
  if ((e = launch_indexer_prefill(true, 128, q_idx, k_idx, w_idx, s->cu_seqlens, s->idx_heads,
                                  at<int2>(ws, L.sched16), counts, 0, L.nb16, seqoff, 0, scores,
                                  at<float2>(ws, L.rowrange), st)) != hipSuccess ||
      (e = launch_kl_lse(q, k, s->cu_seqlens, s->q_heads, s->kv_heads, s->softmax_scale, at<int2>(ws, L.sched128),
                         counts + 1, L.nb128, at<float>(ws, K.lse), st)) != hipSuccess ||
      (e = launch_kl_target(q, k, s->cu_seqlens, s->q_heads, s->kv_heads, s->softmax_scale,
                            at<int2>(ws, L.sched128), counts + 1, L.nb128, s->max_seqlen, at<float>(ws, K.lse), seqoff,
                            P, st)) != hipSuccess ||
      (e = launch_kl_rows(scores, P, seqoff, s->cu_seqlens, s->num_seqs, s->total_tokens,
                          at<float2>(ws, L.rowrange), kl, st)) != hipSuccess ||
      (e = launch_kl_dq(s->idx_heads, static_cast<const uint8_t*>(q_idx), static_cast<const uint8_t*>(k_idx), w_idx,
                        P, seqoff, s->cu_seqlens, at<int2>(ws, K.schedR), counts + 2, K.nbR, dq_idx, dw_idx,
                        st)) != hipSuccess ||
      (e = launch_kl_dk(s->idx_heads, static_cast<const uint8_t*>(q_idx), static_cast<const uint8_t*>(k_idx), w_idx,
                        P, seqoff, s->cu_seqlens, s->num_seqs, at<int2>(ws, K.sched256), counts + 3, K.nb256,
                        s->max_seqlen, s->total_tokens, at<float>(ws, K.dkpart), dk_idx, st)) != hipSuccess)
    return hip_status(e);
  return DSA_OK;
}

int dsa_sparse_attention_fwd_lse(const dsa_prefill_shape* s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* topk_idx, uint16_t* out, float* lse, void* stream) {
  int rc = check_prefill(s, false);
  if (rc) return rc;
  if (s->total_tokens == 0) return DSA_OK;
  if (!q || !k || !v || !topk_idx || !out || !lse) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return DSA_ERR_INVALID_ARGUMENT;
  return hip_status(launch_gather_attention(q, k, v, topk_idx, s->topk, 0, s->cu_seqlens, s->num_seqs, nullptr, 0,
                                            s->total_tokens, s->q_heads, s->kv_heads, s->softmax_scale, 1 << 30, 1,
                                            out, nullptr, nullptr, static_cast<hipStream_t>(stream), lse));
}

int dsa_sparse_attention_bwd_workspace_size(const dsa_prefill_shape* s, size_t* bytes) {
  if (!bytes) return DSA_ERR_INVALID_ARGUMENT;
  int rc = check_prefill(s, false);
  if (rc) return rc;
  if (!dedup_supported(s)) return DSA_ERR_UNSUPPORTED;
  *bytes = bwd_layout(s).total;
  return DSA_OK;
}

int dsa_sparse_attention_bwd(const dsa_prefill_shape* s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const int32_t* topk_idx, const uint16_t* out, const float* lse, const uint16_t* d_out,
                             float* dq, float* dk, float* dv, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_prefill(s, false);
  if (rc) return rc;
  if (!dedup_supported(s)) return DSA_ERR_UNSUPPORTED;
  if (s->total_tokens == 0) return DSA_OK;
  if (!q || !k || !v || !topk_idx || !out || !lse || !d_out || !dq || !dk || !dv || !ws)
    return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(d_out) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(ws))
    return DSA_ERR_INVALID_ARGUMENT;
  const BwdWs W = bwd_layout(s);
  if (ws_bytes < W.total) return DSA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int* counts = at<int>(ws, W.counts);
  const int32_t* cu = s->cu_seqlens;
  float* Dl = at<float>(ws, W.delta);
  uint16_t *qh = at<uint16_t>(ws, W.qh), *kh = at<uint16_t>(ws, W.kh), *vh = at<uint16_t>(ws, W.vh),
           *doh = at<uint16_t>(ws, W.doh), *qt = at<uint16_t>(ws, W.qt), *dot = at<uint16_t>(ws, W.dot);
  float* stats = at<float>(ws, W.stats);
  hipError_t e;
  if ((e = launch_build_schedule(cu, s->num_seqs, 16, W.nb16, at<int2>(ws, W.sched16), counts, nullptr, st)) !=
          hipSuccess ||
      (e = launch_build_schedule(cu, s->num_seqs, 32, W.nb32, at<int2>(ws, W.sched32), counts + 1, nullptr, st)) !=
          hipSuccess ||
      (e = launch_build_schedule(cu, s->num_seqs, 128, W.nb128, at<int2>(ws, W.sched128), counts + 2, nullptr, st)) !=
          hipSuccess ||
      (e = launch_bwd_delta(d_out, out, s->total_tokens * s->q_heads, Dl, st)) != hipSuccess ||
      (e = launch_bwd_prep(q, d_out, lse, Dl, cu, s->num_seqs, s->total_tokens, s->q_heads, s->kv_heads, qh, doh,
                           qt, dot, stats, st)) != hipSuccess ||
      (e = launch_to_f16(k, kh, s->total_tokens * s->kv_heads * 128, st)) != hipSuccess ||
      (e = launch_to_f16(v, vh, s->total_tokens * s->kv_heads * 128, st)) != hipSuccess ||
      (e = launch_union(topk_idx, s->topk, cu, at<int2>(ws, W.sched16), counts, W.nb16, W.ustride,
                        at<int32_t>(ws, W.ukeys), at<uint16_t>(ws, W.umask), at<int>(ws, W.ucount), st)) !=
          hipSuccess ||
      (e = launch_dedup_dq(qh, kh, vh, doh, lse, Dl, cu, s->q_heads, s->kv_heads, s->softmax_scale,
                           at<int2>(ws, W.sched16), counts, W.nb16, W.ustride, at<int32_t>(ws, W.ukeys),
                           at<uint16_t>(ws, W.umask), at<int>(ws, W.ucount), dq, s->max_seqlen, st)) != hipSuccess ||
      (e = launch_sel_bitmap(topk_idx, s->topk, cu, at<int2>(ws, W.sched32), counts + 1, W.nb32,
                             at<uint32_t>(ws, W.bitmap), st)) != hipSuccess ||
      (e = launch_sparse_dkv(qh, kh, vh, doh, qt, dot, stats, cu, s->num_seqs, s->q_heads, s->kv_heads,
                             s->softmax_scale, at<int2>(ws, W.sched128), counts + 2, W.nb128,
                             at<uint32_t>(ws, W.bitmap), s->max_seqlen,
                             s->total_tokens, at<float>(ws, W.dkpart), at<float>(ws, W.dvpart), dk, dv, st)) !=
          hipSuccess)
    return hip_status(e);
  return DSA_OK;
}

int dsa_dedup_workspace_size(const dsa_prefill_shape* s, size_t* bytes) {
  if (!bytes) return DSA_ERR_INVALID_ARGUMENT;
  int rc = check_prefill(s, false);
  if (rc) return rc;
  if (!dedup_supported(s)) return DSA_ERR_UNSUPPORTED;
  *bytes = dedup_layout(s).total;
  return DSA_OK;
}

int dsa_sparse_attention_dedup(const dsa_prefill_shape* s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const int32_t* topk_idx, uint16_t* out, void* dws, size_t dws_bytes, void* stream) {
  int rc = check_prefill(s, false);
  if (rc) return rc;
  if (s->total_tokens == 0) return DSA_OK;
  if (!q || !k || !v || !topk_idx || !out) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return DSA_ERR_INVALID_ARGUMENT;
  DedupWs D;
  if ((rc = check_dedup_ws(s, dws, dws_bytes, &D))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_build_schedule(s->cu_seqlens, s->num_seqs, 16, D.nb16, at<int2>(dws, D.sched16),
                                       at<int>(dws, D.counts), nullptr, st);
  if (e != hipSuccess) return hip_status(e);
  return dedup_attention(s, q, k, v, topk_idx, out, at<int2>(dws, D.sched16), at<int>(dws, D.counts), D.nb16, dws, D,
                         st);
}

int dsa_prefill_dedup(const dsa_prefill_shape* s, const void* q_idx, const void* k_idx, const float* w_idx,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int32_t* topk_idx,
                      void* ws, size_t ws_bytes, void* dws, size_t dws_bytes, void* stream, void* const* events) {
  return prefill_impl(s, q_idx, k_idx, w_idx, q, k, v, out, topk_idx, ws, ws_bytes, stream, events, dws, dws_bytes,
                      true);
}

int dense_causal_attention(const dsa_prefill_shape* s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_prefill(s, false);
  if (rc) return rc;
  if (s->total_tokens == 0) return DSA_OK;  // empty batch: nothing to do, pointers may be null
  if (!q || !k || !v || !out) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return DSA_ERR_INVALID_ARGUMENT;
  PrefillWs L;
  if ((rc = check_prefill_ws(s, ws, ws_bytes, &L))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_build_schedule(s->cu_seqlens, s->num_seqs, 128, L.nb128, at<int2>(ws, L.sched128),
                                       at<int>(ws, L.counts) + 1, nullptr, st);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_dense_prefill(q, k, v, at<uint16_t>(ws, L.v16), s->total_tokens, s->cu_seqlens,
                                         s->num_seqs, s->q_heads, s->kv_heads, s->softmax_scale,
                                         at<int2>(ws, L.sched128), at<int>(ws, L.counts) + 1, L.nb128, out, st));
}

int dsa_decode_workspace_size(const dsa_decode_shape* s, size_t* bytes) {
  if (!bytes) return DSA_ERR_INVALID_ARGUMENT;
  int rc = check_decode(s, false);
  if (rc) return rc;
  *bytes = decode_layout(s).total;
  return DSA_OK;
}

int dsa_kv_append(const dsa_decode_shape* s, const void* k_idx_new, const uint16_t* k_new, const uint16_t* v_new,
                  int32_t* cache_lens, void* k_idx_cache, uint16_t* k_cache, uint16_t* v_cache, void* stream) {
  if (!s || s->batch < 1 || s->cache_capacity < 1 || s->idx_dim < 1 || s->kv_heads < 1 || s->head_dim < 1)
    return DSA_ERR_INVALID_ARGUMENT;
  if (s->idx_dtype != DSA_IDX_BF16 && s->idx_dtype != DSA_IDX_FP8_E4M3) return DSA_ERR_INVALID_ARGUMENT;
  if (!k_idx_new || !k_new || !v_new || !cache_lens || !k_idx_cache || !k_cache || !v_cache)
    return DSA_ERR_INVALID_ARGUMENT;
  const int idx_row_bytes = s->idx_dim * (s->idx_dtype == DSA_IDX_BF16 ? 2 : 1);
  const int kv_row_bytes = s->kv_heads * s->head_dim * 2;
  const bool vec = idx_row_bytes % 16 == 0 && kv_row_bytes % 16 == 0 && aligned16(k_idx_new) && aligned16(k_new) &&
                   aligned16(v_new) && aligned16(k_idx_cache) && aligned16(k_cache) && aligned16(v_cache);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* ki = static_cast<const uint8_t*>(k_idx_new);
  const uint8_t* kn = reinterpret_cast<const uint8_t*>(k_new);
  const uint8_t* vn = reinterpret_cast<const uint8_t*>(v_new);
  uint8_t* kic = static_cast<uint8_t*>(k_idx_cache);
  uint8_t* kc = reinterpret_cast<uint8_t*>(k_cache);
  uint8_t* vc = reinterpret_cast<uint8_t*>(v_cache);
  if (vec)
    kv_append_kernel<true><<<s->batch, 256, 0, st>>>(ki, kn, vn, cache_lens, s->cache_capacity, idx_row_bytes,
                                                     kv_row_bytes, kic, kc, vc);
  else
    kv_append_kernel<false><<<s->batch, 256, 0, st>>>(ki, kn, vn, cache_lens, s->cache_capacity, idx_row_bytes,
                                                      kv_row_bytes, kic, kc, vc);
  return hip_status(hipGetLastError());
}

int dsa_decode(const dsa_decode_shape* s, const void* q_idx, const float* w_idx, const uint16_t* q,
               const void* k_idx_cache, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* out,
               int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(s, q_idx, w_idx, q, k_idx_cache, k_cache, v_cache, out, topk_idx, ws, ws_bytes, stream, nullptr);
}

int dsa_decode_timed(const dsa_decode_shape* s, const void* q_idx, const float* w_idx, const uint16_t* q,
                     const void* k_idx_cache, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* out,
                     int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream, void* const* events) {
  if (!events) return DSA_ERR_INVALID_ARGUMENT;
  return decode_impl(s, q_idx, w_idx, q, k_idx_cache, k_cache, v_cache, out, topk_idx, ws, ws_bytes, stream, events);
}

// Address of this device's copy of `scratch` (looked up once per device, with it current).
static int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return DSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!ptr || !aligned16(ptr)) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

int dsa_decode_noalloc(const dsa_decode_shape* s, const void* q_idx, const float* w_idx, const uint16_t* q,
                       const void* k_idx_cache, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* out,
                       int32_t* topk_idx, void* stream) {
  int rc = check_decode(s, true);
  if (rc) return rc;
  const size_t need = decode_layout(s).total;
  if (need > kDecodeScratchBytes) return DSA_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  return decode_impl(s, q_idx, w_idx, q, k_idx_cache, k_cache, v_cache, out, topk_idx, ws, kDecodeScratchBytes,
                     stream, nullptr);
}

int dense_decode_attention(const dsa_decode_shape* s, const uint16_t* q, const uint16_t* k_cache,
                           const uint16_t* v_cache, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_decode(s, false);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !out || !ws) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(ws))
    return DSA_ERR_INVALID_ARGUMENT;
  const DecodeWs L = decode_layout(s);
  if (ws_bytes < L.total) return DSA_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(launch_gather_attention(q, k_cache, v_cache, nullptr, s->topk, 1, nullptr, 0, s->cache_lens,
                                            s->cache_capacity, s->batch, s->q_heads, s->kv_heads, s->softmax_scale,
                                            kDecodeDenseSplit, L.nsplit_dense, out, at<float>(ws, L.opart),
                                            at<float2>(ws, L.mlpart), static_cast<hipStream_t>(stream)));
}

int dsa_topk(const float* scores, int64_t rows, int32_t n, int64_t ld, const int32_t* row_lens, int32_t k,
             int32_t* out, void* stream) {
  if (rows < 0 || rows > 0x7FFFFFFF || n < 0 || k < 1 || k > (1 << 24)) return DSA_ERR_INVALID_ARGUMENT;
  if (rows == 0) return DSA_OK;
  if (!out || (n > 0 && (!scores || ld < n))) return DSA_ERR_INVALID_ARGUMENT;
  if (rows * (int64_t)k > (int64_t(1) << 40)) return DSA_ERR_UNSUPPORTED;
  return hip_status(launch_topk_general(scores, rows, n, n > 0 ? ld : 0, row_lens, k, out,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
