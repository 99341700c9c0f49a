// decode.hip -- one decode step of DSA (lightning indexer, top-k selection, sparse MLA in MQA
// mode and the merge of its split partials) in a single launch ("DeepSeek-V3.2 技术报告摘要",
// section 1: the indexer scores every preceding token, the fine-grained selection keeps the
// top-k, and MLA in MQA mode attends over the selected entries only).
//
// A decode batch has few rows, so every stage after the key stream is latency-bound and a
// launch boundary between stages costs as much as the stage.  Here the stages are roles of
// the workgroups of one grid, taken in the order the workgroups start (each draws its role
// from an atomic counter when it starts):
//   1. indexer (R x C workgroups): score a contiguous chunk of a row's keys (indexer_core.h),
//      publish the chunk's scores, leading-digit histogram and candidates (topk_select.h) and
//      count the chunk in the row's arrival counter;
//   2. attention (R x S workgroups): load the row's query block, wait for the row's chunks,
//      select the row's top-k from the publications, attend over this split's slots
//      (mla_core.h) and publish the split's partial;
//   3. merge (R x 16 workgroups, only when S > 1): wait for the row's splits and merge them.
// A workgroup only waits for workgroups of an earlier stage, whose roles were drawn before its
// own: those have started, hold their CU and never wait for later roles, so every wait ends
// whatever the number of CUs.  Waits are bounded all the same (a breached contract, such as a
// workspace whose counters are not zero, ends them with a flag instead of a hang).
// Values that cross workgroups are stored with agent scope (written through the L2) and
// published with a release; the counters are left at zero for the next call.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "indexer_core.h"
#include "mla_core.h"
#include "topk_select.h"

namespace dsa {

// Every role runs in 512-thread workgroups (the attention's 8 waves of 16 heads) with the
// whole 160 KB of LDS.  The indexer role streams fp8 keys through 4-slot rings, bf16 keys
// through 3-slot rings, and stages its chunk's scores in the LDS after the rings.
constexpr int kDecThreads = kMlaThreads;
constexpr int kDecLds = 160 * 1024;
template <bool FP8>
using DecIdx = IdxShape<FP8, kDecThreads / kWave, FP8 ? 4 : 3>;
template <bool FP8>
constexpr int kDecMaxSpan = (kDecLds - DecIdx<FP8>::kCoreBytes) / 4;
constexpr int kDecMergeHeads = kDecThreads / kWave;   // heads per merge workgroup (64 threads each)
constexpr uint32_t kSpinLimit = 1u << 22;             // polls of a wait before it gives up

struct DecodeArgs {
  RowsDev rows;
  int R, C, gpb, S, per, k, cached;
  // indexer
  const uint8_t *q_idx;
  const float *q_scale;
  const uint8_t *k_idx;
  const float *k_scale;
  const float *w;
  float *logits;
  int64_t ld;
  int32_t *idx;
  // attention
  const uint16_t *q;
  const uint8_t *kv;
  float scale_log2;
  uint16_t *out;
  float *lse;
  uint16_t *part_o;
  float *part_lse;
  // workspace
  SelWs sel;              // publications and the rows' chunk arrival counters
  uint32_t *ctl;          // [0] next role to draw, [1] waits that gave up (sticky)
  uint32_t *arrive_mla;   // [R] splits of the row published
  uint32_t *arrive_comb;  // [R] merge workgroups of the row past their wait
};

// Waits (thread 0) until *p >= target; false if it gave up.
__device__ __forceinline__ bool wait_count(const uint32_t *p, uint32_t target, uint32_t *err) {
  uint32_t n = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(4);
    if (++n == kSpinLimit) {
      __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
  return true;
}
__device__ __forceinline__ void st_zero(uint32_t *p) {
  __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool FP8, bool PAGED>
__device__ __forceinline__ void decode_index(const DecodeArgs &a, uint8_t *smem, int r, int c) {
  using I = DecIdx<FP8>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int len = a.rows.row_len[r];
  const int n_row_groups = (len + I::kKeys - 1) / I::kKeys;
  const int mine = max(0, min(a.gpb, n_row_groups - c * a.gpb));
  const int ng = wave < mine ? (mine - wave + I::kWaves - 1) / I::kWaves : 0;
  const int span = a.gpb * I::kKeys;
  const int lo = c * span, hi = min(len, lo + span);
  uint8_t *tail = smem + I::kCoreBytes;
  float *sc = reinterpret_cast<float *>(tail);
  index_groups<FP8, PAGED, I::kWaves, I::kDepth, false>(
      smem, a.rows, r, a.q_idx, a.q_scale, a.k_idx, a.k_scale, a.w, tail, (int64_t)c * a.gpb + wave,
      I::kWaves, ng, a.cached != 0, [&](int64_t s, float v) { sc[s - lo] = v; });
  __syncthreads();   // the chunk's scores are in LDS; the query block and the rings are free
  publish_chunk<kDecThreads>(sc, reinterpret_cast<uint32_t *>(smem + I::kQBytes),
                             *reinterpret_cast<PublishLds *>(smem), a.sel, r, c, lo, hi, len,
                             a.logits + (int64_t)r * a.ld, len > a.k);
}

template <bool PAGED>
__device__ __forceinline__ void decode_attend(const DecodeArgs &a, uint8_t *smem, int r, int split,
                                              int span) {
  constexpr int H = kHeadsPerBlock;
  bf16x8 qf[18];
  mla_load_q(a.q, r, qf);   // in flight while the row's chunks finish
  if (threadIdx.x == 0) wait_count(a.sel.arrive + r, (uint32_t)a.C, a.ctl + 1);
  __syncthreads();   // the publications are read with agent-scope loads: no acquire fence
  // the row's top-k, in the tile ring (free until the first tile load)
  using L = SelectLds<kDecThreads>;
  static_assert(sizeof(L) + sizeof(int32_t) * kMaxSlotsPerSplit <= sizeof(MlaShared::tiles),
                "the selection fits the tile ring");
  MlaShared &sh = *reinterpret_cast<MlaShared *>(smem);
  int32_t *lst = reinterpret_cast<int32_t *>(smem + sizeof(L));
  const int len = a.rows.row_len[r];
  select_published<kDecThreads>(a.sel, r, len, a.k, span, a.logits + (int64_t)r * a.ld, lst,
                                *reinterpret_cast<L *>(smem));
  __syncthreads();
  const int slot_begin = split * a.per;
  const int n_slots = max(0, min(a.k, slot_begin + a.per) - slot_begin);
  int sv[kSlotRounds];
  int32_t *idx_row = a.idx + (int64_t)r * a.k + slot_begin;
#pragma unroll
  for (int j = 0; j < kSlotRounds; ++j) {
    const int t = j * kMlaThreads + threadIdx.x;
    sv[j] = t < n_slots ? lst[slot_begin + t] : -1;
    if (t < n_slots) idx_row[t] = sv[j];
  }
  __syncthreads();   // the list is read before the ring takes tiles
  const int n_valid = mla_resolve_slots<PAGED>(sh, sv, n_slots, a.rows, r);
  const bool one = a.S == 1;
  const int64_t po = ((int64_t)r * a.S + split) * H;
  mla_attend(sh, qf, n_valid, a.kv, a.scale_log2,
             one ? a.out + (int64_t)r * H * kDv : a.part_o + po * kDv,
             one ? (a.lse ? a.lse + (int64_t)r * H : nullptr) : a.part_lse + po, one ? kLn2 : 1.f,
             !one);
  if (one) {
    if (threadIdx.x == 0) st_zero(a.sel.arrive + r);   // the row's only reader is done with it
    return;
  }
  // publish the partial; the row's last split also leaves the chunk counter at zero
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old =
        __hip_atomic_fetch_add(a.arrive_mla + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)a.S - 1) st_zero(a.sel.arrive + r);
  }
}

__device__ __forceinline__ void decode_merge(const DecodeArgs &a, int r, int hg) {
  constexpr int H = kHeadsPerBlock;
  constexpr int G = H / kDecMergeHeads;
  if (threadIdx.x == 0) wait_count(a.arrive_mla + r, (uint32_t)a.S, a.ctl + 1);
  __syncthreads();   // the partials are read with agent-scope loads: no acquire fence
  const int h = hg * kDecMergeHeads + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  mla_combine_head<true>(a.S, H, h, d0, a.part_o + (int64_t)r * a.S * H * kDv,
                   a.part_lse + (int64_t)r * a.S * H, a.out + ((int64_t)r * H + h) * kDv,
                   a.lse ? a.lse + (int64_t)r * H + h : nullptr, a.lse && (threadIdx.x & 63) == 0);
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(a.arrive_comb + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == G - 1) {   // every merge workgroup of the row is past its wait
      st_zero(a.arrive_mla + r);
      st_zero(a.arrive_comb + r);
    }
  }
}

template <bool FP8, bool PAGED>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dec_smem[];
  constexpr int G = kHeadsPerBlock / kDecMergeHeads;
  const uint32_t n_index = (uint32_t)a.R * a.C, n_attend = (uint32_t)a.R * a.S;
  const uint32_t total = n_index + n_attend + (a.S > 1 ? (uint32_t)a.R * G : 0u);
  uint32_t *bc = reinterpret_cast<uint32_t *>(dec_smem);
  if (threadIdx.x == 0) {
    const uint32_t id = __hip_atomic_fetch_add(a.ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (id == total - 1) st_zero(a.ctl);   // every role is drawn: ready for the next call
    bc[0] = id;
  }
  __syncthreads();
  const uint32_t id = bc[0];
  __syncthreads();
  if (id < n_index) {
    decode_index<FP8, PAGED>(a, dec_smem, (int)(id / a.C), (int)(id % a.C));
  } else if (id < n_index + n_attend) {
    const uint32_t j = id - n_index;
    decode_attend<PAGED>(a, dec_smem, (int)(j / a.S), (int)(j % a.S),
                         a.gpb * DecIdx<FP8>::kKeys);
  } else if (id < total) {
    const uint32_t j = id - n_index - n_attend;
    decode_merge(a, (int)(j / G), (int)(j % G));
  }
}

// ------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------
namespace {

struct DecShape {
  int C, gpb, cap, S, per;
};

DecShape decode_shape(int num_rows, int max_row_len, bool fp8, int k) {
  DecShape d;
  const int waves = kDecThreads / kWave;
  const int keys = fp8 ? DecIdx<true>::kKeys : DecIdx<false>::kKeys;
  const int max_span = fp8 ? kDecMaxSpan<true> : kDecMaxSpan<false>;
  // about 256 indexer workgroups, whole 64-key multiples per wave, the chunk within the LDS
  const int64_t total = (int64_t)num_rows * max_row_len;
  int64_t kpw = (total + (int64_t)waves * 256 - 1) / ((int64_t)waves * 256);
  kpw = ((kpw + 63) / 64) * 64;
  if (kpw < 64) kpw = 64;
  const int64_t lim = (int64_t)(max_span / waves) / 64 * 64;
  if (kpw > lim) kpw = lim;
  const int64_t span = waves * kpw;
  d.gpb = (int)(span / keys);
  d.C = (int)((max_row_len + span - 1) / span);
  int tpl = kDecThreads;
  while (tpl > 1 && tpl * d.C > kDecThreads) tpl >>= 1;
  const int want = max(256, (4 * k + d.C - 1) / d.C);
  int cap = 16;
  while (cap < want) cap <<= 1;
  const int cap_lim = kSelCandPerThread * tpl < 1024 ? kSelCandPerThread * tpl : 1024;
  if (cap > cap_lim) cap = cap_lim;
  if (cap < tpl) cap = tpl;
  d.cap = cap;
  d.S = mla_num_splits(num_rows, kHeadsPerBlock, k);
  d.per = (((k + d.S - 1) / d.S) + kTile - 1) / kTile * kTile;
  return d;
}

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool decode_onelaunch_ok(int num_rows, int max_row_len, bool fp8, int k) {
  if (num_rows < 1 || num_rows > 256 || max_row_len > kMaxChunks * kChunk || k > kMaxSlotsPerSplit)
    return false;
  const DecShape d = decode_shape(num_rows, max_row_len, fp8, k);
  return d.C >= 1 && d.C <= kMaxChunks && d.C <= kDecThreads && d.S <= kMaxCombine;
}

size_t decode_onelaunch_ws_bytes(int num_rows, int max_row_len, bool fp8, int k) {
  const DecShape d = decode_shape(num_rows, max_row_len, fp8, k);
  const size_t parts = d.S > 1 ? (size_t)num_rows * d.S * kHeadsPerBlock * (kDv * 2 + 4) : 0;
  return a256(64 * 4) + 2 * a256(4 * (size_t)num_rows) + a256(sel_ws_bytes(num_rows, d.C, d.cap)) +
         parts;
}

hipError_t launch_decode_onelaunch(const RowsHost &rh, bool paged, bool fp8, const void *q_idx,
                                   const float *q_scale, const void *k_idx, const float *k_scale,
                                   const float *w, float *logits, int64_t ld, int topk,
                                   int32_t *idx, float scale, const void *q, const void *kv,
                                   void *out, float *lse, void *ws, hipStream_t stream) {
  const DecShape d = decode_shape(rh.num_rows, rh.max_row_len, fp8, topk);
  const int R = rh.num_rows;
  DecodeArgs a;
  a.rows = RowsDev{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  a.R = R;
  a.C = d.C;
  a.gpb = d.gpb;
  a.S = d.S;
  a.per = d.per;
  a.k = topk;
  a.cached = rh.num_rows > rh.num_seqs;
  a.q_idx = static_cast<const uint8_t *>(q_idx);
  a.q_scale = q_scale;
  a.k_idx = static_cast<const uint8_t *>(k_idx);
  a.k_scale = k_scale;
  a.w = w;
  a.logits = logits;
  a.ld = ld;
  a.idx = idx;
  a.q = static_cast<const uint16_t *>(q);
  a.kv = static_cast<const uint8_t *>(kv);
  a.scale_log2 = scale * kLog2e;
  a.out = static_cast<uint16_t *>(out);
  a.lse = lse;
  uint8_t *p = static_cast<uint8_t *>(ws);
  a.ctl = reinterpret_cast<uint32_t *>(p);
  p += a256(64 * 4);
  a.arrive_mla = reinterpret_cast<uint32_t *>(p);
  p += a256(4 * (size_t)R);
  a.arrive_comb = reinterpret_cast<uint32_t *>(p);
  p += a256(4 * (size_t)R);
  a.sel = carve_sel_ws(p, R, d.C, d.cap);
  p += a256(sel_ws_bytes(R, d.C, d.cap));
  a.part_o = reinterpret_cast<uint16_t *>(p);
  a.part_lse = reinterpret_cast<float *>(p + (size_t)R * d.S * kHeadsPerBlock * kDv * 2);
  constexpr int G = kHeadsPerBlock / kDecMergeHeads;
  const unsigned grid = (unsigned)(R * d.C + R * d.S + (d.S > 1 ? R * G : 0));
  static std::atomic<uint64_t> lds_set[4];
  const int which = (fp8 ? 2 : 0) + (paged ? 1 : 0);
  hipError_t e;
  auto go = [&](auto kernel) {
    e = ensure_dynamic_lds(kernel, kDecLds, lds_set[which]);
    if (e != hipSuccess) return;
    kernel<<<grid, kDecThreads, kDecLds, stream>>>(a);
    e = hipGetLastError();
  };
  if (fp8) {
    if (paged) go(&decode_kernel<true, true>);
    else go(&decode_kernel<true, false>);
  } else {
    if (paged) go(&decode_kernel<false, true>);
    else go(&decode_kernel<false, false>);
  }
  return e;
}

}  // namespace dsa
