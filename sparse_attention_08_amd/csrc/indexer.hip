// indexer.hip -- lightning-indexer scores on gfx950.
//
// I[t,s] = sum_j w[t,j] * ReLU(q[t,j,:] . k[s,:]) over the preceding tokens s of the
// query's sequence ("DeepSeek-V3.2 技术报告摘要", section 1, DSA ① Lightning Indexer:
// a few indexer heads, one key per token shared by all heads, FP8 supported).
//
// The MFMA kernel (the streaming core of indexer_core.h) serves every batch shape of fp8 keys
// and the bf16 batches with few rows per sequence (decode, multi-token decode);
// indexer_prefill.hip shares key tiles between rows for bf16 prefill.  Its SEL variant also
// selects each row's top-k inside the launch (topk_select.h).
#include "dsa_device.h"
#include "dsa_launch.h"
#include "indexer_core.h"
#include "topk_select.h"

namespace dsa {

// ------------------------------------------------------------------------------------
// fp32 path (any small H, D): one thread per key, plain fp32 FMA.  This is the
// exactness path (checked at 1e-5 relative) and is not tuned.
// ------------------------------------------------------------------------------------
template <bool PAGED>
__global__ __launch_bounds__(256) void indexer_f32_kernel(RowsDev rows, int H, int D,
                                                          const float *__restrict__ q,
                                                          const float *__restrict__ k,
                                                          const float *__restrict__ w,
                                                          float *__restrict__ logits, int64_t ld) {
  extern __shared__ float smem[];   // q row [H*D] then w row [H]
  const int r = blockIdx.y;
  const int len = rows.row_len[r];
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if ((int64_t)blockIdx.x * blockDim.x >= len) return;
  float *qs = smem;
  float *ws = smem + H * D;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) qs[i] = q[(int64_t)r * H * D + i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) ws[i] = w[(int64_t)r * H + i];
  __syncthreads();
  if (s >= len) return;
  const int b = rows.row_seq[r];
  const float *kr = k + cache_row<PAGED>(rows, b, s) * D;
  float acc = 0.f;
  for (int j = 0; j < H; ++j) {
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot = fmaf(qs[j * D + d], kr[d], dot);
    acc = fmaf(ws[j], fmaxf(dot, 0.f), acc);
  }
  logits[(int64_t)r * ld + s] = acc;
}

hipError_t launch_indexer_f32(const RowsHost &rh, bool paged, int H, int D, const float *q,
                              const float *k, const float *w, float *logits, int64_t ld,
                              hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  dim3 grid((rh.max_row_len + 255) / 256, rh.num_rows);
  size_t shm = sizeof(float) * ((size_t)H * D + H);
  if (paged)
    indexer_f32_kernel<true><<<grid, 256, shm, stream>>>(rows, H, D, q, k, w, logits, ld);
  else
    indexer_f32_kernel<false><<<grid, 256, shm, stream>>>(rows, H, D, q, k, w, logits, ld);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// MFMA path, 64 heads x 128 dims, bf16 or OCP e4m3.
// ------------------------------------------------------------------------------------
// Launch shape (measured on MI355X): fp8 keys with 16 waves per workgroup and 2-slot rings,
// bf16 keys (more registers per wave) with 8 waves and 3-slot rings; the grid is sized for
// about 256 workgroups.
#ifndef DSA_IDX_WAVES_FP8
#define DSA_IDX_WAVES_FP8 16
#endif
#ifndef DSA_IDX_DEPTH_FP8
#define DSA_IDX_DEPTH_FP8 2
#endif
#ifndef DSA_IDX_WAVES_BF16
#define DSA_IDX_WAVES_BF16 8
#endif
#ifndef DSA_IDX_DEPTH_BF16
#define DSA_IDX_DEPTH_BF16 3
#endif
#ifndef DSA_IDX_BLOCKS
#define DSA_IDX_BLOCKS 256
#endif

template <bool FP8>
using IdxCfg = IdxShape<FP8, FP8 ? DSA_IDX_WAVES_FP8 : DSA_IDX_WAVES_BF16,
                        FP8 ? DSA_IDX_DEPTH_FP8 : DSA_IDX_DEPTH_BF16>;
// With SEL the workgroup's chunk of scores is staged in the LDS left after the core.
template <bool FP8>
constexpr int kSelMaxSpan = (160 * 1024 - IdxCfg<FP8>::kCoreBytes) / 4;

// SEL: the workgroups of a row also select the row's top-k.  Workgroup c then scores the
// contiguous chunk of groups [c*gpb, (c+1)*gpb) of its row (its waves take them round-robin)
// into LDS; publish_chunk writes the scores out, hands the chunk's histogram and candidates
// to the row's last workgroup to finish, which runs the exact selection (select_published) and
// writes idx.  Without SEL the row's groups are dealt to all its waves round-robin (wave wr of
// WR takes groups wr, wr + WR, ...), so at any time the row's waves stream one contiguous
// window of it, and the scores are stored as they are made.
struct IdxSel {
  SelWs ws;
  int gpb;        // key groups per workgroup
  int k;
  int32_t *idx;   // [R, k]
};

template <bool FP8, bool PAGED, bool SEL>
__global__ __launch_bounds__(IdxCfg<FP8>::kThreads) void indexer_mfma_kernel(
    RowsDev rows, const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const uint8_t *__restrict__ k, const float *__restrict__ k_scale, const float *__restrict__ w,
    float *__restrict__ logits, int64_t ld, int cached, IdxSel sel) {
  using C = IdxCfg<FP8>;
  extern __shared__ __attribute__((aligned(16))) uint8_t idx_smem[];
  uint8_t *smem = idx_smem;
  const int r = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int len = rows.row_len[r];
  const int n_row_groups = (len + C::kKeys - 1) / C::kKeys;
  float *out = logits + (int64_t)r * ld;
  // past the core: the chunk's scores (SEL), or the head weights
  uint8_t *tail = smem + C::kCoreBytes;
  if constexpr (SEL) {
    const int mine = max(0, min(sel.gpb, n_row_groups - (int)blockIdx.x * sel.gpb));
    const int ng = wave < mine ? (mine - wave + C::kWaves - 1) / C::kWaves : 0;
    const int span = sel.gpb * C::kKeys;
    const int lo = blockIdx.x * span, hi = min(len, lo + span);
    float *sc = reinterpret_cast<float *>(tail);
    index_groups<FP8, PAGED, C::kWaves, C::kDepth, false>(
        smem, rows, r, q, q_scale, k, k_scale, w, tail, (int64_t)blockIdx.x * sel.gpb + wave,
        C::kWaves, ng, cached != 0, [&](int64_t s, float v) { sc[s - lo] = v; });
    __syncthreads();   // the chunk's scores are in LDS; the query block and the rings are free
    PublishLds &pl = *reinterpret_cast<PublishLds *>(smem);
    if (!publish_chunk<C::kThreads>(sc, reinterpret_cast<uint32_t *>(smem + C::kQBytes), pl, sel.ws, r,
                                    blockIdx.x, lo, hi, len, out, len > sel.k))
      return;
    __syncthreads();   // the publication scratch is reused by the selection
    if (threadIdx.x == 0)   // every workgroup of the row has counted itself: ready for the next call
      __hip_atomic_store(sel.ws.arrive + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    select_published<C::kThreads>(sel.ws, r, len, sel.k, span, out, sel.idx + (int64_t)r * sel.k,
                                  *reinterpret_cast<SelectLds<C::kThreads> *>(smem));
  } else {
    const int waves_per_row = gridDim.x * C::kWaves;
    const int wr = blockIdx.x * C::kWaves + wave;
    if (blockIdx.x * C::kWaves >= n_row_groups) return;   // uniform over the workgroup
    const int ng = wr < n_row_groups ? (n_row_groups - wr + waves_per_row - 1) / waves_per_row : 0;
    index_groups<FP8, PAGED, C::kWaves, C::kDepth, true>(
        smem, rows, r, q, q_scale, k, k_scale, w, tail, wr, waves_per_row, ng, cached != 0,
        [&](int64_t s, float v) { out[s] = v; });
  }
}

template <bool FP8>
static size_t lds_bytes(bool sel) {
  using C = IdxCfg<FP8>;
  static_assert(C::kRingBytes >= (int)sizeof(uint32_t) * kLeadBins,
                "the histogram fits the ring area");
  static_assert(sizeof(SelectLds<C::kThreads>) <= 160 * 1024, "the selection fits the LDS");
  static_assert(kSelMaxSpan<FP8> >= 128, "room for the head weights");
  if (!sel) return (size_t)C::kCoreBytes + 512;
  return 160 * 1024;
}
size_t indexer_lds_bytes(bool fp8, bool sel) { return fp8 ? lds_bytes<true>(sel) : lds_bytes<false>(sel); }

template <bool FP8, bool PAGED, bool SEL>
static hipError_t launch_one(dim3 grid, size_t shm, hipStream_t stream, const RowsDev &rows,
                             const uint8_t *q8, const float *q_scale, const uint8_t *k8,
                             const float *k_scale, const float *w, float *logits, int64_t ld,
                             int cached, const IdxSel &sel) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = ensure_dynamic_lds(&indexer_mfma_kernel<FP8, PAGED, SEL>, (int)shm, lds_set);
  if (e != hipSuccess) return e;
  indexer_mfma_kernel<FP8, PAGED, SEL><<<grid, IdxCfg<FP8>::kThreads, shm, stream>>>(
      rows, q8, q_scale, k8, k_scale, w, logits, ld, cached, sel);
  return hipGetLastError();
}

// One workgroup per CU at a time (the LDS rings fill most of the CU's 160 KB); the keys per
// wave are sized for about DSA_IDX_BLOCKS workgroups in all, whole 64-key multiples.  With
// the in-kernel selection a workgroup's chunk of scores must also fit its LDS.
static int64_t keys_per_wave(int num_rows, int max_row_len, bool fp8, bool sel) {
  const int64_t total = (int64_t)num_rows * max_row_len;
  constexpr int64_t kBlocksTarget = DSA_IDX_BLOCKS;
  const int64_t waves = fp8 ? IdxCfg<true>::kWaves : IdxCfg<false>::kWaves;
  int64_t kpw = (total + waves * kBlocksTarget - 1) / (waves * kBlocksTarget);
  kpw = ((kpw + 63) / 64) * 64;
  if (kpw < 64) kpw = 64;
  // at most 64 groups per wave (one page id per lane)
  int64_t max_kpw = 64 * (fp8 ? IdxCfg<true>::kKeys : IdxCfg<false>::kKeys);
  if (sel) {
    const int64_t span = fp8 ? kSelMaxSpan<true> : kSelMaxSpan<false>;
    const int64_t lim = (span / waves) / 64 * 64;
    if (lim < max_kpw) max_kpw = lim;
  }
  return kpw > max_kpw ? max_kpw : kpw;
}

static int blocks_per_row(int num_rows, int max_row_len, bool fp8, bool sel) {
  const int64_t per_block = (fp8 ? IdxCfg<true>::kWaves : IdxCfg<false>::kWaves) *
                            keys_per_wave(num_rows, max_row_len, fp8, sel);
  return (int)((max_row_len + per_block - 1) / per_block);
}
int indexer_blocks_per_row(int num_rows, int max_row_len, bool fp8) {
  return blocks_per_row(num_rows, max_row_len, fp8, false);
}

// Candidates kept per chunk for the in-kernel selection: about four times a chunk's share of
// k (at least 256), at most kSelCandPerThread per selecting thread and at most 1024.
int indexer_sel_cap(int num_rows, int max_row_len, bool fp8, int k) {
  const int C = blocks_per_row(num_rows, max_row_len, fp8, true);
  const int nt = fp8 ? IdxCfg<true>::kThreads : IdxCfg<false>::kThreads;
  int tpl = nt;
  while (tpl > 1 && tpl * C > nt) tpl >>= 1;
  const int want = max(256, (4 * k + C - 1) / C);
  int cap = 16;
  while (cap < want) cap <<= 1;
  const int lim = kSelCandPerThread * tpl < 1024 ? kSelCandPerThread * tpl : 1024;
  if (cap > lim) cap = lim;
  if (cap < tpl) cap = tpl;
  return cap;
}

bool indexer_sel_ok(int num_rows, int max_row_len, bool fp8) {
  // decode-shaped batches (the selection runs once per row inside the grid)
  if (num_rows < 1 || num_rows > 256 || max_row_len > kMaxChunks * kChunk) return false;
  const int C = blocks_per_row(num_rows, max_row_len, fp8, true);
  const int nt = fp8 ? IdxCfg<true>::kThreads : IdxCfg<false>::kThreads;
  return C >= 1 && C <= kMaxChunks && C <= nt;
}

size_t indexer_sel_ws_bytes(int num_rows, int max_row_len, bool fp8, int k) {
  return sel_ws_bytes(num_rows, blocks_per_row(num_rows, max_row_len, fp8, true),
                      indexer_sel_cap(num_rows, max_row_len, fp8, k));
}

template <bool SEL>
static hipError_t launch_indexer(const RowsHost &rh, bool paged, bool fp8, const void *q,
                                 const float *q_scale, const void *k, const float *k_scale,
                                 const float *w, float *logits, int64_t ld, const IdxSel &sel,
                                 hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  dim3 grid((unsigned)blocks_per_row(rh.num_rows, rh.max_row_len, fp8, SEL), rh.num_rows);
  const size_t shm = indexer_lds_bytes(fp8, SEL);
  const uint8_t *q8 = static_cast<const uint8_t *>(q);
  const uint8_t *k8 = static_cast<const uint8_t *>(k);
  const int cached = rh.num_rows > rh.num_seqs;   // rows share sequences: keep keys in cache
  if (fp8)
    return paged ? launch_one<true, true, SEL>(grid, shm, stream, rows, q8, q_scale, k8, k_scale, w, logits, ld, cached, sel)
                 : launch_one<true, false, SEL>(grid, shm, stream, rows, q8, q_scale, k8, k_scale, w, logits, ld, cached, sel);
  return paged ? launch_one<false, true, SEL>(grid, shm, stream, rows, q8, q_scale, k8, k_scale, w, logits, ld, cached, sel)
               : launch_one<false, false, SEL>(grid, shm, stream, rows, q8, q_scale, k8, k_scale, w, logits, ld, cached, sel);
}

hipError_t launch_indexer_mfma(const RowsHost &rh, bool paged, bool fp8, const void *q,
                               const float *q_scale, const void *k, const float *k_scale,
                               const float *w, float *logits, int64_t ld, hipStream_t stream) {
  return launch_indexer<false>(rh, paged, fp8, q, q_scale, k, k_scale, w, logits, ld, IdxSel{},
                               stream);
}

hipError_t launch_indexer_select(const RowsHost &rh, bool paged, bool fp8, const void *q,
                                 const float *q_scale, const void *k, const float *k_scale,
                                 const float *w, float *logits, int64_t ld, int topk,
                                 int32_t *idx, void *ws, hipStream_t stream) {
  IdxSel sel;
  const int C = blocks_per_row(rh.num_rows, rh.max_row_len, fp8, true);
  sel.ws = carve_sel_ws(ws, rh.num_rows, C, indexer_sel_cap(rh.num_rows, rh.max_row_len, fp8, topk));
  const int64_t per_block = (fp8 ? IdxCfg<true>::kWaves : IdxCfg<false>::kWaves) *
                            keys_per_wave(rh.num_rows, rh.max_row_len, fp8, true);
  sel.gpb = (int)(per_block / (fp8 ? IdxCfg<true>::kKeys : IdxCfg<false>::kKeys));
  sel.k = topk;
  sel.idx = idx;
  return launch_indexer<true>(rh, paged, fp8, q, q_scale, k, k_scale, w, logits, ld, sel, stream);
}

}  // namespace dsa
