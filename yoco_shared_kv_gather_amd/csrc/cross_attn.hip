// yoco_cross_attn: one YOCO cross layer's attention over the shared paged cache.
//
// What is computed ("KV cache memory systems", section "Cache contents";
// "YOCO_论文与推理数据流详解" §10.4 and §13.2): every request has one query per
// query head, and it attends to the request's whole context of K^/V^ rows in
// the one cache that all cross layers share; each logical block of the
// context is found through the block table ("KV cache memory systems",
// section "Contiguous allocation wastes capacity").
//
// How (gfx950):
//   * Split-KV.  A workgroup of four wavefronts owns one work item =
//     (request, KV head, partition of `partition_tokens` context tokens), so a
//     long context still spreads over every compute unit.  The partition's
//     block-table slice is staged in LDS once; the four wavefronts take every
//     fourth iteration of the partition and combine their softmax states in
//     LDS at the end.
//   * When a request has more than one partition, each workgroup writes an
//     unnormalised partial (acc, running max m, running sum l) to the
//     workspace and a second, small kernel merges them with log-sum-exp
//     weights in partition order (deterministic).  A request that fits one
//     partition is finished by the first kernel.  The kernel boundary makes
//     the partials visible; making them visible from inside the first kernel
//     would need an agent-scope release (an L2 write-back) per workgroup,
//     and those serialise per XCD.
//   * Each K^/V^ row is read once and used for all G query heads of its KV
//     group (GQA); the G queries are staged in LDS.
//   * A row of head_dim elements is split into 16-byte chunks; LPR lanes cover
//     one row with CPL chunks each, so one wavefront load instruction reads
//     64/LPR rows, coalesced within each cache block.  The next iteration's
//     rows are loaded while the current ones are used (two register sets).
//   * q.k uses v_dot2_f32_bf16 (two bf16 products per instruction, fp32
//     accumulation) and a DPP all-reduce over the LPR lanes of a row.
//   * Online softmax in base 2 with a lazy maximum: the running max of a row
//     group is raised only when a score exceeds it by more than 2^8, so the
//     accumulators are rescaled rarely; sums stay within 256x the true terms.
//   * p.v in fp32 FMA; bf16 values widen with one shift or mask.
//
// yoco_cross_attn_varlen generalises the query side ("You Only Cache Once, in
// vLLM", section "Implementation in vLLM": the cross-decoder metadata keeps
// seq_lens and marks attention causal, so a request with q logits rows has
// queries at its last q positions; Gemma 3n's sliding-window cross layers read
// a shared sliding-window cache, same page, section "Gemma 3n"):
//   * a window of W tokens restricts the query at position p to keys
//     p-W < j <= p.  With one query per request this only moves the start of
//     the range the partitions cover, so the decode kernel is unchanged.
//   * several query rows per request: a work item carries QPI consecutive
//     query rows of one request (QPI*G <= 8 "virtual heads" share every K^/V^
//     row), and each row masks the keys outside its own causal window.

#include <cmath>
#include <map>
#include <mutex>
#include <utility>

#include "yoco_internal.h"

namespace {

using yoco::bf16_hi;
using yoco::bf16_lo;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMaxSlack = 8.0f;      // log2 of the largest un-rescaled term
constexpr float kInitMax = -1.0e30f;       // finite "minus infinity" for running maxima
constexpr int kWaves = 4;                  // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSliceBlocks = 512;       // block-table entries one partition may span
constexpr int kMaxQueueSeqs = 2048;        // requests the persistent schedule's LDS prefix holds
constexpr int kQueueLineWords = 32;        // the two queue counters sit on separate 128-byte lines
constexpr int64_t kQueueHeaderBytes = 2048; // queue counters, the rest reserved
static_assert(kQueueHeaderBytes == YOCO_CROSS_ATTN_QUEUE_BYTES, "queue header size");

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* out;
  float* ws_acc;        // [num_seqs][Hq][num_parts][D]
  float* ws_ml;         // [num_seqs][Hq][num_parts][2]  (max, sum), base-2 units
  uint32_t* queue;      // persistent schedule: fetch counters, then done counters; nullptr otherwise
  int64_t block_stride; // elements per physical block (Hkv * bs * D)
  int32_t head_stride;  // elements per KV head inside a block (bs * D)
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t block_size;
  int32_t bs_shift;
  int32_t max_blocks;
  int32_t len_cap;      // seq_lens are clamped to [0, len_cap]
  int32_t part_tokens;
  int32_t num_parts;
  float scale_log2;     // scale * log2(e)
  uint32_t flags;
  const int32_t* qsl;   // query_start_loc [num_seqs+1] (several query rows per request), nullptr otherwise
  int32_t num_rows;     // query rows of q and out (num_seqs without qsl)
  int32_t max_qlen;     // query rows per request are clamped to this (1 without qsl)
  int32_t window;       // sliding window in tokens; 0 = the whole context
};

// First context position any query of a request can see: its queries sit at
// positions n-ql .. n-1, and with a window of W tokens the earliest key of the
// first one is n-ql-W+1 (without a window, position 0).
__host__ __device__ inline int range_lo(int n, int ql, int window) {
  if (window <= 0) return 0;
  const int lo = n - ql - window + 1;
  return lo > 0 ? lo : 0;
}

template <bool kBf16, int D>
struct Layout {
  static constexpr int kEpc = kBf16 ? 8 : 4;              // elements per 16-byte chunk
  static constexpr int kChunks = D / kEpc;                // chunks per row
  static constexpr int kLpr = kChunks / 2 < 16 ? kChunks / 2 : 16;   // lanes per row
  static constexpr int kCpl = kChunks / kLpr;             // chunks per lane
  static constexpr int kRpw = 64 / kLpr;                  // rows per wave instruction
  static constexpr int kU = 2;                            // row sets per iteration
  static constexpr int kIterTokens = kRpw * kU;
};

// Dot product of one 16-byte chunk of q with one of k, accumulated into acc.
template <bool kBf16>
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k, float acc);

template <>
__device__ __forceinline__ float chunk_dot<true>(const uint4& q, const uint4& k, float acc) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k.x), __builtin_bit_cast(bf2, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k.y), __builtin_bit_cast(bf2, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k.z), __builtin_bit_cast(bf2, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k.w), __builtin_bit_cast(bf2, q.w), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<false>(const uint4& q, const uint4& k, float acc) {
  acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
  return acc;
}

// Element e of a 16-byte chunk as fp32.
template <bool kBf16>
__device__ __forceinline__ float chunk_elem(const uint4& c, int e) {
  const uint32_t w = e < (kBf16 ? 2 : 1) ? c.x : e < (kBf16 ? 4 : 2) ? c.y : e < (kBf16 ? 6 : 3) ? c.z : c.w;
  if constexpr (kBf16) {
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  } else {
    return __uint_as_float(w);
  }
}

// 2^x with the hardware instruction (no denormal range reduction): the
// softmax terms here are 2^(s - m) with s - m <= 8, and terms below 2^-126
// flushed to zero change no output bit that matters next to the max term.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v + (v of another lane chosen by a DPP control word), in every lane.
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
  const int other = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, true);
  return v + __builtin_bit_cast(float, other);
}

// Sum over aligned groups of kLanes lanes (4, 8 or 16), result in every lane.
// quad_perm [1,0,3,2] and [2,3,0,1] pair lanes inside a quad; row_half_mirror
// pairs each quad of 8 lanes with the other; row_mirror pairs the two halves
// of a 16-lane row.
template <int kLanes>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(kLanes == 4 || kLanes == 8 || kLanes == 16, "group of 4, 8 or 16 lanes");
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  if constexpr (kLanes >= 8) v = dpp_add<0x141>(v);
  if constexpr (kLanes >= 16) v = dpp_add<0x140>(v);
  return v;
}

// Partitions of a context of n tokens: ceil(n/P) pieces of P tokens (the
// last one shorter; an empty context has one, empty, partition).  For the
// schedule they fall in two groups: the leading n/P - 1 partitions when
// n >= 2P ("big"), and the last one or two ("small"), which hold the short
// piece.  All big items are scheduled before all small ones, so the work ends
// on the short pieces.
__host__ __device__ inline int big_parts(int n, int P) {
  const int nb = n / P;
  return nb >= 2 ? nb - 1 : 0;
}
__host__ __device__ inline int small_parts(int n, int P) {
  return n <= 0 ? 1 : (n - big_parts(n, P) * P + P - 1) / P;
}
__host__ __device__ inline int parts_of(int n, int P) { return big_parts(n, P) + small_parts(n, P); }

// Merge the partials of one (query row, query head):
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// One workgroup per (request, query row of the request, head); rows past the
// request's query count return at once.  256 threads: thread t owns the
// float4 slice (t % (D/4)) of head_dim and partitions
// p = t / (D/4) + k * (256 / (D/4)).  Each thread sums its partitions relative
// to their own maximum, so the partial loads need not wait for the global
// one; the groups are then rescaled and added in group order through LDS
// (deterministic).  Rows whose context fits one partition were finished by
// the first kernel.
template <int D>
__global__ __launch_bounds__(kThreads) void cross_attn_merge_kernel(AttnArgs a) {
  constexpr int kSlices = D / 4;                 // float4 slices of a head
  constexpr int kGroups = kThreads / kSlices;    // partition groups
  __shared__ float4 s_num[kGroups][kSlices];
  __shared__ float s_den[kGroups];
  __shared__ float s_max[kGroups];
  const int64_t per_req = static_cast<int64_t>(a.max_qlen) * a.num_q_heads;
  const int r = static_cast<int>(blockIdx.x / per_req);
  const int rem = static_cast<int>(blockIdx.x - r * per_req);
  const int qi = rem / a.num_q_heads;
  const int h = rem - qi * a.num_q_heads;
  const int tid = threadIdx.x;
  int n = a.seq_lens[r];
  n = n < 0 ? 0 : (n > a.len_cap ? a.len_cap : n);
  int ql = 1, row = r;
  if (a.qsl != nullptr) {
    const int qb = min(max(a.qsl[r], 0), a.num_rows);
    const int qe = min(max(a.qsl[r + 1], 0), a.num_rows);
    ql = min(max(qe - qb, 0), a.max_qlen);
    row = qb + qi;
  }
  if (qi >= ql) return;
  const int np = parts_of(n - range_lo(n, ql, a.window), a.part_tokens);
  if (np <= 1) return;
  const int64_t rh = static_cast<int64_t>(row) * a.num_q_heads + h;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + rh * a.num_parts;
  const float4* acc = reinterpret_cast<const float4*>(a.ws_acc + rh * a.num_parts * D);
  const int slice = tid % kSlices;
  const int grp = tid / kSlices;

  float m_loc = kInitMax;
#pragma unroll 8
  for (int p = grp; p < np; p += kGroups) m_loc = fmaxf(m_loc, ml[p].x);
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float den = 0.0f;
#pragma unroll 8
  for (int p = grp; p < np; p += kGroups) {
    const float2 part = ml[p];
    const float4 v = acc[static_cast<int64_t>(p) * kSlices + slice];
    const float w = exp2f(part.x - m_loc);
    den = fmaf(w, part.y, den);
    num.x = fmaf(w, v.x, num.x);
    num.y = fmaf(w, v.y, num.y);
    num.z = fmaf(w, v.z, num.z);
    num.w = fmaf(w, v.w, num.w);
  }
  s_num[grp][slice] = num;
  if (slice == 0) {
    s_den[grp] = den;
    s_max[grp] = m_loc;
  }
  __syncthreads();
  if (tid < kSlices) {
    float mx = s_max[0];
#pragma unroll
    for (int g2 = 1; g2 < kGroups; ++g2) mx = fmaxf(mx, s_max[g2]);
    float4 t = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float dsum = 0.0f;
#pragma unroll
    for (int g2 = 0; g2 < kGroups; ++g2) {
      const float f = exp2f(s_max[g2] - mx);
      const float4 u = s_num[g2][tid];
      t.x = fmaf(f, u.x, t.x);
      t.y = fmaf(f, u.y, t.y);
      t.z = fmaf(f, u.z, t.z);
      t.w = fmaf(f, u.w, t.w);
      dsum = fmaf(f, s_den[g2], dsum);
    }
    const float inv = dsum == 0.0f ? 0.0f : 1.0f / dsum;
    reinterpret_cast<float4*>(a.out + rh * D)[tid] = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  }
}

template <bool kBf16, int D>
struct RowSet {
  uint4 k[Layout<kBf16, D>::kU][Layout<kBf16, D>::kCpl];
  uint4 v[Layout<kBf16, D>::kU][Layout<kBf16, D>::kCpl];
  bool valid[Layout<kBf16, D>::kU];
  int pos[Layout<kBf16, D>::kU];     // logical position of the row (masks of the several-query path)
};

// Shared memory of one workgroup: block-table slices and queries of the
// current and the next work item (double buffered), the per-wavefront softmax
// states and, for the persistent schedule, every request's clamped length,
// (several-query path) its first query row, and the prefix of work-item
// counts.  VG = query vectors per item (G heads times the rows per item).
template <bool kBf16, int D, int VG, bool kVar>
struct AttnSmem {
  static constexpr int kQChunks = VG * D * (kBf16 ? 2 : 4) / 16;   // 16-byte chunks of an item's queries
  int32_t blocks[2][kMaxSliceBlocks];
  uint4 q[2][kQChunks];
  float acc[kWaves][VG][D];
  float ml[kWaves][VG][2];
  int32_t len[kMaxQueueSeqs];
  int32_t qs[kVar ? kMaxQueueSeqs + 1 : 1];
  int32_t pref[kMaxQueueSeqs + 1];
  int32_t pref2[kMaxQueueSeqs + 1];
  int32_t wsum[2 * kWaves];
  uint32_t next;
};

// One work item: query heads g*G .. g*G+G-1 of request r (context length n)
// over context tokens [start, end), which span block-table entries
// first_blk .. first_blk+num_blk-1.  The request's partitions cover
// [lo, n).  Several-query path: the item's query rows are row0 ..
// row0+nq-1, the first of them at logical position pbase (decode path: row0
// = r, nq = 1).  `valid` is false past the last item.
struct Item {
  bool valid;
  int r, g, part, n, lo, start, end, first_blk, num_blk;
  int row0, nq, pbase;
};

// The fields are the same in every lane (the inputs come from LDS or from
// ballots): readfirstlane keeps them in scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ Item make_item(const AttnArgs& a, bool valid, int r, int g, int part, int n, int lo,
                                          int row0, int nq, int pbase) {
  Item it;
  it.valid = valid;
  it.r = valid ? uniform(r) : 0;
  it.g = valid ? uniform(g) : 0;
  it.part = valid ? uniform(part) : 0;
  it.n = valid ? uniform(n) : 0;
  it.lo = valid ? uniform(lo) : 0;
  it.row0 = valid ? uniform(row0) : 0;
  it.nq = valid ? uniform(nq) : 0;
  it.pbase = valid ? uniform(pbase) : 0;
  it.start = it.lo + it.part * a.part_tokens;
  it.end = min(it.start + a.part_tokens, it.n);
  // An item without rows stages (harmlessly) the first table entry of its
  // row: its start may lie past the row's last entry.
  it.first_blk = it.end > it.start ? it.start >> a.bs_shift : 0;
  it.num_blk = it.end > it.start ? ((it.end - 1) >> a.bs_shift) - it.first_blk + 1 : 0;
  return it;
}

// Largest r in [0, R) with pref[r] <= k, for pref non-decreasing with
// pref[0] = 0 <= k < pref[R]: each step tests 64 evenly spaced candidates
// with one ballot, so R <= 4096 takes two steps.  Wave-uniform result.
__device__ __forceinline__ int find_request(const int32_t* pref, int R, uint32_t k) {
  const int lane = threadIdx.x & 63;
  int lo = 0, span = R;
  while (span > 1) {
    const int stride = (span + 63) >> 6;
    const int off = lane * stride;
    const bool le = off < span && static_cast<uint32_t>(pref[lo + min(off, span - 1)]) <= k;
    const unsigned long long mask = __ballot(le);
    const int j = 63 - __clzll(mask);
    const int nlo = lo + j * stride;
    span = min(stride, lo + span - nlo);
    lo = nlo;
  }
  return lo;
}

// Work items are (request, KV head, [query-row group,] partition).  Two
// schedules:
//   * persistent (a.queue != nullptr): as many workgroups as fit on the GPU at
//     once.  Items are numbered request by request, counting only the
//     partitions that hold tokens (an empty context has one item, which
//     writes its zero rows), so no workgroup is spent on an empty partition.
//     Workgroup w starts with item w (no atomic on the critical path at the
//     start); after that every workgroup takes the next unclaimed item from
//     one device-wide counter, so a workgroup that
//     runs faster (the XCDs do not all get the same share of HBM bandwidth)
//     takes more items.  The last workgroup to finish
//     resets the counter to zero: it knows it is last from a second (done)
//     counter, and every workgroup's final fetch has returned before it
//     counts itself done, so no fetch can follow the reset.  Same-line
//     atomics serialise, so the two counters sit on separate 128-byte lines.
//   * one item per workgroup (decode path with more requests than the LDS
//     prefix holds): (request, KV head) varies fastest; the hardware deals
//     consecutive workgroups to the eight XCDs in turn, so every XCD gets an
//     even share of the partitions that hold tokens, and the empty tail
//     partitions of short requests come last.
// Items are pipelined: near the end of an item's stream the next item's index
// is fetched and its block-table slice and queries are loaded into registers;
// the last iteration requests the next item's first rows, and when the stream
// ends the slice and queries go to the other LDS buffer while the finished
// item's wavefronts are combined and written.
//
// QPI = 0: one query row per request (row r), every head of an item sees the
// item's whole range.  QPI >= 1: QPI query rows of one request per item, each
// with its own causal (and window) limits.
template <bool kBf16, int D, int G, int QPI>
__global__ __launch_bounds__(kThreads) void cross_attn_kernel(AttnArgs a) {
  using L = Layout<kBf16, D>;
  constexpr bool kVar = QPI > 0;
  constexpr int kQ = kVar ? QPI : 1;                               // query rows per item
  constexpr int VG = G * kQ;                                       // query vectors per item
  using Smem = AttnSmem<kBf16, D, VG, kVar>;
  constexpr int kEpc = L::kEpc, kLpr = L::kLpr, kCpl = L::kCpl, kRpw = L::kRpw, kU = L::kU;
  constexpr int kIterTokens = L::kIterTokens;
  constexpr int kElemBytes = kBf16 ? 2 : 4;
  constexpr int kQChunks = Smem::kQChunks;
  constexpr int kHeadChunks = D * kElemBytes / 16;                 // 16-byte chunks of one query vector
  constexpr int kTblPer = kMaxSliceBlocks / kThreads;               // table entries per thread
  constexpr int kQPer = (kQChunks + kThreads - 1) / kThreads;       // query chunks per thread
  static_assert(kMaxSliceBlocks % kThreads == 0, "slice staging");
  static_assert(VG <= 8, "at most eight query vectors per item");

  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int row = lane / kLpr;
  const int cl = lane % kLpr;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool reverse = (a.flags & YOCO_FLAG_REVERSE_ORDER) != 0;
  const bool persistent = a.queue != nullptr;
  const int R = a.num_seqs;
  uint32_t* fetch_ctr = a.queue;
  uint32_t* done_ctr = persistent ? a.queue + kQueueLineWords : nullptr;
  uint32_t total = 0, total_big = 0;

  // Query rows of request r (several-query path), clamped to max_qlen.
  auto qlen_of = [&](int r) -> int {
    if constexpr (kVar) {
      return min(max(sm.qs[r + 1] - sm.qs[r], 0), a.max_qlen);
    } else {
      return 1;
    }
  };

  if (persistent) {
    // Clamped lengths (and first query rows), then the exclusive prefixes of
    // the big items (pref) and of the small items (pref2) per request: all
    // big items are numbered before all small ones.
    for (int i = tid; i < R; i += kThreads) {
      const int n = a.seq_lens[i];
      sm.len[i] = n < 0 ? 0 : (n > a.len_cap ? a.len_cap : n);
    }
    if constexpr (kVar) {
      for (int i = tid; i <= R; i += kThreads) sm.qs[i] = min(max(a.qsl[i], 0), a.num_rows);
    }
    __syncthreads();
    const int per = (R + kThreads - 1) / kThreads;
    const int lo = min(tid * per, R);
    const int hi = min(lo + per, R);
    auto counts = [&](int i, int& nb, int& ns) {
      const int n = sm.len[i];
      const int ql = qlen_of(i);
      const int m = n - range_lo(n, ql, a.window);
      const int groups = kVar ? (ql + kQ - 1) / kQ : 1;
      nb = big_parts(m, a.part_tokens) * a.num_kv_heads * groups;
      ns = small_parts(m, a.part_tokens) * a.num_kv_heads * groups;
    };
    int local_b = 0, local_s = 0;
    for (int i = lo; i < hi; ++i) {
      int nb, ns;
      counts(i, nb, ns);
      local_b += nb;
      local_s += ns;
    }
    int incl_b = local_b, incl_s = local_s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int tb = __shfl_up(incl_b, off, 64);
      const int ts = __shfl_up(incl_s, off, 64);
      if (lane >= off) {
        incl_b += tb;
        incl_s += ts;
      }
    }
    if (lane == 63) {
      sm.wsum[wave] = incl_b;
      sm.wsum[kWaves + wave] = incl_s;
    }
    __syncthreads();
    int run_b = incl_b - local_b, run_s = incl_s - local_s;
    for (int w = 0; w < wave; ++w) {
      run_b += sm.wsum[w];
      run_s += sm.wsum[kWaves + w];
    }
    for (int i = lo; i < hi; ++i) {
      sm.pref[i] = run_b;
      sm.pref2[i] = run_s;
      int nb, ns;
      counts(i, nb, ns);
      run_b += nb;
      run_s += ns;
    }
    if (tid == kThreads - 1) {
      sm.pref[R] = run_b;
      sm.pref2[R] = run_s;
    }
    __syncthreads();
    total_big = static_cast<uint32_t>(uniform(sm.pref[R]));
    total = total_big + static_cast<uint32_t>(uniform(sm.pref2[R]));
  }

  // Item number k of the persistent schedule.  Within a request, the KV head
  // varies fastest, then the query-row group, then the partition.
  auto item_at = [&](uint32_t k) -> Item {
    if (k >= total) return make_item(a, false, 0, 0, 0, 0, 0, 0, 0, 0);
    const uint32_t kk = reverse ? total - 1u - k : k;
    const bool big = kk < total_big;
    const int32_t* pref = big ? sm.pref : sm.pref2;
    const uint32_t j = big ? kk : kk - total_big;
    const int r = find_request(pref, R, j);
    const int idx = static_cast<int>(j - static_cast<uint32_t>(pref[r]));
    const int n = sm.len[r];
    const int ql = qlen_of(r);
    const int lo = range_lo(n, ql, a.window);
    const int groups = kVar ? (ql + kQ - 1) / kQ : 1;
    const int per = max(a.num_kv_heads * groups, 1);
    const int sub = idx / per;
    const int rem = idx - sub * per;
    const int qgrp = rem / a.num_kv_heads;
    const int g = rem - qgrp * a.num_kv_heads;
    const int part = big ? sub : big_parts(n - lo, a.part_tokens) + sub;
    if constexpr (kVar) {
      return make_item(a, true, r, g, part, n, lo, sm.qs[r] + qgrp * kQ, min(kQ, ql - qgrp * kQ),
                       n - ql + qgrp * kQ);
    } else {
      return make_item(a, true, r, g, part, n, lo, r, 1, n - 1);
    }
  };

  // Block-table slice and queries of an item: loaded into registers (indices
  // clamped into the slice, so the loads need no branch), then stored to LDS.
  // Each lane also keeps the block ids of the rows it reads first in that
  // item (and the item's first block), so those rows can be requested before
  // the slice is in LDS.
  int32_t st_tbl[kTblPer];
  uint4 st_q[kQPer];
  int32_t st_nb[kU];
  int32_t st_nb0;
  auto valid_block = [&](int b) { return static_cast<unsigned>(b) < static_cast<unsigned>(a.num_blocks) ? b : -1; };
  auto stage_load = [&](const Item& it) {
    const int32_t* row_table = a.block_table + static_cast<int64_t>(it.r) * a.max_blocks;
    const int32_t* table = row_table + it.first_blk;
    const int last = it.num_blk > 0 ? it.num_blk - 1 : 0;
#pragma unroll
    for (int j = 0; j < kTblPer; ++j) st_tbl[j] = table[min(tid + j * kThreads, last)];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = it.start + wave_u * kIterTokens + u * kRpw + row;
      st_nb[u] = valid_block(row_table[j < it.end ? (j >> a.bs_shift) : it.first_blk]);
    }
    st_nb0 = valid_block(table[0]);
    if constexpr (kVar) {
      // Query vector v = i*G + h is head g*G+h of row row0+i; rows past the
      // item's nq repeat its last row (loaded, never used).
#pragma unroll
      for (int j = 0; j < kQPer; ++j) {
        const int c = min(tid + j * kThreads, kQChunks - 1);
        const int v = c / kHeadChunks;
        const int i = v / G;
        const int qrow = it.row0 + max(0, min(i, it.nq - 1));
        const uint4* qg = reinterpret_cast<const uint4*>(
            static_cast<const char*>(a.q) +
            ((static_cast<int64_t>(qrow) * a.num_q_heads + it.g * G + (v - i * G)) * D) * kElemBytes);
        st_q[j] = qg[c - v * kHeadChunks];
      }
    } else {
      const uint4* qg = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                       (static_cast<int64_t>(it.r) * a.num_q_heads + it.g * G) * D *
                                                           kElemBytes);
#pragma unroll
      for (int j = 0; j < kQPer; ++j) st_q[j] = qg[min(tid + j * kThreads, kQChunks - 1)];
    }
  };
  auto stage_store = [&](const Item& it, int buf) {
#pragma unroll
    for (int j = 0; j < kTblPer; ++j) {
      const int i = tid + j * kThreads;
      if (i < it.num_blk) sm.blocks[buf][i] = valid_block(st_tbl[j]);
    }
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      const int i = tid + j * kThreads;
      if (i < kQChunks) sm.q[buf][i] = st_q[j];
    }
  };

  // Loads are unconditional (no branch around them, so the next iteration's
  // loads stay in flight while the current rows are used).  A row past the
  // end of the item, or in an out-of-range block, reads the item's first row
  // instead (block 0 if that block is out of range too) and is masked: its
  // score is -inf and its values are zeroed.  Only items with rows
  // (num_blk > 0) are ever loaded.
  auto load = [&](RowSet<kBf16, D>& rs, const Item& it, int buf, int iter) {
    const char* kb = static_cast<const char*>(a.k) + static_cast<int64_t>(it.g) * a.head_stride * kElemBytes;
    const char* vb = static_cast<const char*>(a.v) + static_cast<int64_t>(it.g) * a.head_stride * kElemBytes;
    const int off_mask = a.block_size - 1;
    const int b0 = sm.blocks[buf][0];
    const int64_t dummy_off =
        (static_cast<int64_t>(b0 >= 0 ? b0 : 0) * a.block_stride + static_cast<int64_t>(it.start & off_mask) * D) *
        kElemBytes;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = it.start + iter * kIterTokens + u * kRpw + row;
      const bool in_range = j < it.end;
      const int blk = sm.blocks[buf][((in_range ? j : it.start) >> a.bs_shift) - it.first_blk];
      rs.valid[u] = in_range && blk >= 0;
      rs.pos[u] = j;
      const int64_t off = rs.valid[u] ? (static_cast<int64_t>(blk) * a.block_stride +
                                         static_cast<int64_t>(j & off_mask) * D) * kElemBytes
                                      : dummy_off;
#pragma unroll
      for (int i = 0; i < kCpl; ++i) {
        const int64_t c = off + static_cast<int64_t>((cl + kLpr * i) * kEpc) * kElemBytes;
        rs.k[u][i] = *reinterpret_cast<const uint4*>(kb + c);
        rs.v[u][i] = *reinterpret_cast<const uint4*>(vb + c);
      }
    }
  };

  // Rows of one iteration of a wavefront: iteration `iter` of item `it`
  // (slice in LDS buffer `buf`), or, once iter reaches num_iters, the
  // wavefront's first rows of item `nx` (block ids from the staging
  // registers).  One branch-free set of loads either way.
  auto load_step = [&](RowSet<kBf16, D>& rs, const Item& it, int buf, int iter, int num_iters, const Item& nx) {
    const bool to_nx = iter >= num_iters;
    const int g = to_nx ? nx.g : it.g;
    const char* kb = static_cast<const char*>(a.k) + static_cast<int64_t>(g) * a.head_stride * kElemBytes;
    const char* vb = static_cast<const char*>(a.v) + static_cast<int64_t>(g) * a.head_stride * kElemBytes;
    const int off_mask = a.block_size - 1;
    const int start = to_nx ? nx.start : it.start;
    const int end = to_nx ? nx.end : it.end;
    const int b0 = to_nx ? st_nb0 : sm.blocks[buf][0];
    const int64_t dummy_off =
        (static_cast<int64_t>(b0 >= 0 ? b0 : 0) * a.block_stride + static_cast<int64_t>(start & off_mask) * D) *
        kElemBytes;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = (to_nx ? nx.start + wave_u * kIterTokens : it.start + iter * kIterTokens) + u * kRpw + row;
      const bool in_range = j < end;
      const int lds_blk = sm.blocks[buf][((in_range && !to_nx ? j : it.start) >> a.bs_shift) - it.first_blk];
      const int blk = to_nx ? st_nb[u] : lds_blk;
      rs.valid[u] = in_range && blk >= 0;
      rs.pos[u] = j;
      const int64_t off = rs.valid[u] ? (static_cast<int64_t>(blk) * a.block_stride +
                                         static_cast<int64_t>(j & off_mask) * D) * kElemBytes
                                      : dummy_off;
#pragma unroll
      for (int i = 0; i < kCpl; ++i) {
        const int64_t c = off + static_cast<int64_t>((cl + kLpr * i) * kEpc) * kElemBytes;
        rs.k[u][i] = *reinterpret_cast<const uint4*>(kb + c);
        rs.v[u][i] = *reinterpret_cast<const uint4*>(vb + c);
      }
    }
  };

  float acc[VG][kCpl][kEpc];
  float m[VG], lsum[VG];
  // Several-query path: keys [qlo[i], qhi[i]) are visible to the item's
  // query row i (its causal limit and window); empty for rows past nq.
  int qlo[kQ], qhi[kQ];
  auto set_limits = [&](const Item& it) {
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
      const int p = it.pbase + i;
      qhi[i] = i < it.nq ? p + 1 : 0;
      qlo[i] = a.window > 0 ? p - a.window + 1 : 0;
    }
  };

  auto compute = [&](const RowSet<kBf16, D>& rs, int buf) {
    float s[kU][VG];
#pragma unroll
    for (int h = 0; h < VG; ++h) {
      uint4 qh[kCpl];
#pragma unroll
      for (int i = 0; i < kCpl; ++i) qh[i] = sm.q[buf][(h * D + (cl + kLpr * i) * kEpc) * kElemBytes / 16];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < kCpl; ++i) t = chunk_dot<kBf16>(qh[i], rs.k[u][i], t);
        t = group_sum<kLpr>(t);
        bool ok = rs.valid[u];
        if constexpr (kVar) {
          const int qi = h / G;
          ok = ok && rs.pos[u] >= qlo[qi] && rs.pos[u] < qhi[qi];
        }
        s[u][h] = ok ? t * a.scale_log2 : -INFINITY;
      }
    }
    // Lazy running maximum per row group and head.
#pragma unroll
    for (int h = 0; h < VG; ++h) {
      float cand = s[0][h];
#pragma unroll
      for (int u = 1; u < kU; ++u) cand = fmaxf(cand, s[u][h]);
      if (cand > m[h] + kLazyMaxSlack) {
        const float corr = fast_exp2(m[h] - cand);
        lsum[h] *= corr;
#pragma unroll
        for (int i = 0; i < kCpl; ++i)
#pragma unroll
          for (int e = 0; e < kEpc; ++e) acc[h][i][e] *= corr;
        m[h] = cand;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float p[VG];
#pragma unroll
      for (int h = 0; h < VG; ++h) {
        p[h] = fast_exp2(s[u][h] - m[h]);
        lsum[h] += p[h];
      }
#pragma unroll
      for (int i = 0; i < kCpl; ++i) {
        // A masked row (p = 0) read some other row, which may hold NaN:
        // zero its values so that it adds exactly nothing.
        const uint4 vc = rs.valid[u] ? rs.v[u][i] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int e = 0; e < kEpc; ++e) {
          const float x = chunk_elem<kBf16>(vc, e);
#pragma unroll
          for (int h = 0; h < VG; ++h) acc[h][i][e] = fmaf(p[h], x, acc[h][i][e]);
        }
      }
    }
  };

  // The first item (workgroup w starts with item w; the persistent schedule
  // fetches the next one while it runs).
  Item cur, nxt;
  bool nxt_known = !persistent;
  if (persistent) {
    cur = item_at(blockIdx.x);
    nxt = cur;
  } else {
    const uint32_t items = static_cast<uint32_t>(R) * a.num_kv_heads * a.num_parts;
    const uint32_t item = reverse ? items - 1u - blockIdx.x : blockIdx.x;
    const uint32_t pairs = static_cast<uint32_t>(R) * a.num_kv_heads;
    const int part = static_cast<int>(item / pairs);
    const uint32_t rg = item % pairs;
    const int r = static_cast<int>(rg / a.num_kv_heads);
    int n = a.seq_lens[r];
    n = n < 0 ? 0 : (n > a.len_cap ? a.len_cap : n);
    cur = make_item(a, true, r, static_cast<int>(rg % a.num_kv_heads), part, n, range_lo(n, 1, a.window), r, 1,
                    n - 1);
    nxt = make_item(a, false, 0, 0, 0, 0, 0, 0, 0, 0);
  }

  RowSet<kBf16, D> buf_a, buf_b;
  bool first_in_b = false;                     // the current item's first rows sit in buf_b
  int lb = 0;                                  // LDS buffer of the current item
  if (cur.valid) {
    stage_load(cur);
    stage_store(cur, 0);
    __syncthreads();
    if (cur.num_blk > 0) load(buf_a, cur, 0, wave_u);
  }

  while (cur.valid) {
    const int num_iters = (cur.end - cur.start + kIterTokens - 1) / kIterTokens;
    // The next item is fetched late, so that when the queue runs dry a
    // workgroup holds little more than the item it is streaming: in an item
    // of three or more rounds (a round = one iteration of every wavefront)
    // the fetch is issued three rounds before the end, its result is shared
    // one round later (one barrier) and the next item's staging loads go
    // out then, in time for the last round to request its first rows.  A
    // shorter item fetches at its start.
    const int rounds = num_iters / kWaves;
    const bool late = !nxt_known && rounds >= 3;
    if (!nxt_known && !late) {
      if (tid == 0) sm.next = gridDim.x + atomicAdd(fetch_ctr, 1u);
      __syncthreads();
      nxt = item_at(static_cast<uint32_t>(uniform(static_cast<int>(sm.next))));
      nxt_known = true;
    }
    if (nxt_known) stage_load(nxt);
    if (first_in_b) buf_a = buf_b;
    first_in_b = false;
    uint32_t pending = 0;
    auto late_fetch = [&](int rd) {
      if (!late) return;
      if (rd == rounds - 3 && tid == 0) pending = atomicAdd(fetch_ctr, 1u);
      if (rd == rounds - 2) {
        if (tid == 0) sm.next = gridDim.x + pending;
        __syncthreads();
        nxt = item_at(static_cast<uint32_t>(uniform(static_cast<int>(sm.next))));
        stage_load(nxt);
      }
    };

    if (cur.num_blk > 0) {
      if constexpr (kVar) set_limits(cur);
#pragma unroll
      for (int h = 0; h < VG; ++h) {
        m[h] = kInitMax;
        lsum[h] = 0.0f;
#pragma unroll
        for (int i = 0; i < kCpl; ++i)
#pragma unroll
          for (int e = 0; e < kEpc; ++e) acc[h][i][e] = 0.0f;
      }
      // Wavefront w takes iterations w, w+4, ... (buf_a already holds
      // iteration w); the next one's rows are in flight while the current
      // ones are used.  Past the last iteration the prefetch requests the
      // wavefront's first rows of the next item.
      int it = wave_u;
      int rd = 0;
      while (it < num_iters) {
        late_fetch(rd);
        load_step(buf_b, cur, lb, it + kWaves, num_iters, nxt);
        compute(buf_a, lb);
        it += kWaves;
        ++rd;
        if (it >= num_iters) {
          first_in_b = true;
          break;
        }
        late_fetch(rd);
        load_step(buf_a, cur, lb, it + kWaves, num_iters, nxt);
        compute(buf_b, lb);
        it += kWaves;
        ++rd;
      }

      // Combine the row groups of the wavefront (lanes with the same cl).
#pragma unroll
      for (int mask = kLpr; mask < 64; mask <<= 1) {
#pragma unroll
        for (int h = 0; h < VG; ++h) {
          const float mo = __shfl_xor(m[h], mask, 64);
          const float lo = __shfl_xor(lsum[h], mask, 64);
          const float mx = fmaxf(m[h], mo);
          const float fa = exp2f(m[h] - mx);
          const float fb = exp2f(mo - mx);
          lsum[h] = lsum[h] * fa + lo * fb;
#pragma unroll
          for (int i = 0; i < kCpl; ++i)
#pragma unroll
            for (int e = 0; e < kEpc; ++e) {
              const float other = __shfl_xor(acc[h][i][e], mask, 64);
              acc[h][i][e] = acc[h][i][e] * fa + other * fb;
            }
          m[h] = mx;
        }
      }
      if (row == 0) {
#pragma unroll
        for (int h = 0; h < VG; ++h) {
#pragma unroll
          for (int i = 0; i < kCpl; ++i)
#pragma unroll
            for (int e = 0; e < kEpc; ++e) sm.acc[wave][h][(cl + kLpr * i) * kEpc + e] = acc[h][i][e];
          if (cl == 0) {
            sm.ml[wave][h][0] = m[h];
            sm.ml[wave][h][1] = lsum[h];
          }
        }
      }
    }

    // A wavefront that had no iteration of this item (or an item without
    // rows) has not requested its first rows of the next item yet.
    if (wave_u >= num_iters) load_step(buf_a, cur, lb, num_iters, num_iters, nxt);

    // Hand over to the next item: its slice and queries into the other LDS
    // buffer, then the finished item written.
    if (nxt.valid) stage_store(nxt, lb ^ 1);
    __syncthreads();

    // Output slot of query vector v of the item (-1: a padding row).
    auto out_row = [&](int v) -> int64_t {
      if constexpr (kVar) {
        const int i = v / G;
        return i < cur.nq ? static_cast<int64_t>(cur.row0 + i) * a.num_q_heads + cur.g * G + (v - i * G) : -1;
      } else {
        return static_cast<int64_t>(cur.r) * a.num_q_heads + cur.g * G + v;
      }
    };
    if (cur.num_blk > 0) {
      // Combine the four wavefronts, then finish (one partition) or publish.
      const int np_r = parts_of(cur.n - cur.lo, a.part_tokens);
      for (int e = tid; e < VG * D; e += kThreads) {
        const int h = e / D;
        const int d = e - h * D;
        const int64_t rh = out_row(h);
        if (rh < 0) continue;
        float mx = sm.ml[0][h][0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm.ml[w][h][0]);
        float den = 0.0f, num = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float f = exp2f(sm.ml[w][h][0] - mx);
          den = fmaf(f, sm.ml[w][h][1], den);
          num = fmaf(f, sm.acc[w][h][d], num);
        }
        if (np_r == 1) {
          a.out[rh * D + d] = den == 0.0f ? 0.0f : num / den;
        } else {
          const int64_t slot = rh * a.num_parts + cur.part;
          a.ws_acc[slot * D + d] = num;
          if (d == 0) {
            a.ws_ml[slot * 2] = mx;
            a.ws_ml[slot * 2 + 1] = den;
          }
        }
      }
    } else if (cur.n == 0 && cur.part == 0) {
      // An empty context answers zeros (partitions past the end of a
      // non-empty context, one-item-per-workgroup schedule only, do nothing).
      for (int e = tid; e < VG * D; e += kThreads) {
        const int h = e / D;
        const int64_t rh = out_row(h);
        if (rh >= 0) a.out[rh * D + (e - h * D)] = 0.0f;
      }
    }
    __syncthreads();                           // sm.acc, sm.ml and sm.next are reused

    cur = nxt;
    nxt_known = !persistent;                   // the one-item-per-workgroup schedule stops here
    lb ^= 1;
  }

  if (persistent && tid == 0) {
    const uint32_t d = atomicAdd(done_ctr, 1u);
    if (d == gridDim.x - 1) {
      atomicExch(fetch_ctr, 0u);
      atomicExch(done_ctr, 0u);
    }
  }
}

// ---- host side ---------------------------------------------------------------

constexpr int kMaxParts = 65535;

// Largest partition whose block-table slice fits the LDS staging array.
int32_t max_partition(int32_t block_size) {
  const int64_t cap = static_cast<int64_t>(kMaxSliceBlocks - 1) * block_size / 64 * 64;
  return static_cast<int32_t>(cap < 16384 ? cap : 16384);
}

int32_t resolve_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                          int32_t block_size, int32_t requested) {
  if (requested > 0) return requested;
  const int64_t pairs = static_cast<int64_t>(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
  const int64_t len = max_seq_len > 0 ? max_seq_len : 1;
  const int64_t d = head_dim > 0 ? head_dim : 128;
  int64_t p;
  if (num_seqs <= kMaxQueueSeqs) {
    // Persistent schedule: items of about 512 KB of bf16 K^/V^ (P*D = 2^17:
    // measured best on all four workloads within ~1.5%), but at least about
    // 1024 items when every context is full length (two per resident
    // workgroup) and at most 256 partitions per request, so the merge stays
    // small next to the stream.
    p = yoco::round_up((int64_t{1} << 17) / d, 64);
    const int64_t p_items = yoco::round_up(yoco::ceil_div(len, yoco::ceil_div(1024, pairs)), 64);
    if (p > p_items) p = p_items;
    if (p < 256) p = 256;
    const int64_t p_merge = yoco::round_up(yoco::ceil_div(len, 256), 64);
    if (p < p_merge) p = p_merge;
  } else {
    // One workgroup per item: about 2048 workgroups with partitions of 64
    // tokens or more.
    p = yoco::round_up(yoco::ceil_div(len, yoco::ceil_div(2048, pairs)), 64);
  }
  const int64_t cap = max_partition(block_size > 0 ? block_size : 1);
  if (p > cap) p = cap;
  if (p < 64) p = 64;
  return static_cast<int32_t>(p);
}

int32_t num_partitions(int32_t max_seq_len, int32_t part_tokens) {
  const int64_t np = yoco::ceil_div(max_seq_len > 0 ? max_seq_len : 1, part_tokens);
  return static_cast<int32_t>(np);
}

// Workspace: [work-queue counters, kQueueHeaderBytes][acc fp32 num_seqs*Hq*num_parts*D | pad to 256]
// [ml fp32 num_seqs*Hq*num_parts*2]; the partials only when there is more than one partition.
struct WorkspaceLayout {
  int64_t acc_offset = 0;
  int64_t ml_offset = 0;
  int64_t total = 0;
};

WorkspaceLayout workspace_layout(int32_t num_rows, int32_t num_q_heads, int32_t head_dim, int32_t num_parts) {
  WorkspaceLayout w;
  w.total = kQueueHeaderBytes;
  if (num_parts <= 1) return w;
  const int64_t slots = static_cast<int64_t>(num_rows) * num_q_heads * num_parts;
  w.acc_offset = kQueueHeaderBytes;
  w.ml_offset = yoco::round_up(w.acc_offset + slots * head_dim * 4, 256);
  w.total = w.ml_offset + slots * 2 * 4;
  return w;
}

// Workgroups of one kernel instance resident on the current device at once
// (compute units x workgroups per compute unit), cached per device and kernel.
int resident_workgroups(const void* kernel, int per_cu_query(int*)) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  if (per_cu_query(&per_cu) != 0 || per_cu <= 0) return 0;
  cache[key] = cus * per_cu;
  return cus * per_cu;
}

template <bool kBf16, int D, int G, int QPI>
int per_cu_workgroups(int* out) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, cross_attn_kernel<kBf16, D, G, QPI>, kThreads, 0) ==
                 hipSuccess ? 0 : 1;
}

// Launch the attention kernel: persistent (grid = resident workgroups, at
// most one per work item) when the requests fit the LDS prefix, else one
// workgroup per work item.  Returns false if the occupancy query failed.
template <bool kBf16, int D, int G, int QPI>
bool launch(AttnArgs a, int64_t items, hipStream_t stream) {
  int64_t grid = items;
  if (a.queue != nullptr) {
    const int slots = resident_workgroups(reinterpret_cast<const void*>(cross_attn_kernel<kBf16, D, G, QPI>),
                                          per_cu_workgroups<kBf16, D, G, QPI>);
    if (slots <= 0) return false;
    grid = items < slots ? items : slots;
  }
  hipLaunchKernelGGL((cross_attn_kernel<kBf16, D, G, QPI>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                     stream, a);
  return true;
}

// Query rows per work item: 0 for the decode kernel (one row per request);
// with query_start_loc, 8/G rows (eight query vectors per item) when a request
// may have more than one row, else 1.
template <bool kBf16, int D, int G>
int dispatch_rows(int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  constexpr int kWide = 8 / G;
  if (qpi == 0) return launch<kBf16, D, G, 0>(a, items, stream) ? 1 : -1;
  if (qpi == 1) return launch<kBf16, D, G, 1>(a, items, stream) ? 1 : -1;
  if constexpr (kWide > 1) {
    if (qpi == kWide) return launch<kBf16, D, G, kWide>(a, items, stream) ? 1 : -1;
  }
  return 0;
}

template <bool kBf16, int D>
int dispatch_group(int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  switch (group) {
    case 1: return dispatch_rows<kBf16, D, 1>(qpi, a, items, stream);
    case 2: return dispatch_rows<kBf16, D, 2>(qpi, a, items, stream);
    case 4: return dispatch_rows<kBf16, D, 4>(qpi, a, items, stream);
    case 8: return dispatch_rows<kBf16, D, 8>(qpi, a, items, stream);
    default: return 0;
  }
}

// 1: launched, 0: no kernel for the shape, -1: the occupancy query failed.
template <bool kBf16>
int dispatch_dim(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  switch (head_dim) {
    case 64: return dispatch_group<kBf16, 64>(group, qpi, a, items, stream);
    case 128: return dispatch_group<kBf16, 128>(group, qpi, a, items, stream);
    case 256: return dispatch_group<kBf16, 256>(group, qpi, a, items, stream);
    default: return 0;
  }
}

bool supported_dim(int d) { return d == 64 || d == 128 || d == 256; }

// Length the partitions of the longest context cover: with a window, a
// request's queries see at most window + max_query_len - 1 positions.
int32_t effective_len(int32_t max_seq_len, int32_t max_qlen, int32_t window) {
  if (window <= 0) return max_seq_len;
  const int64_t span = static_cast<int64_t>(window) + (max_qlen > 1 ? max_qlen : 1) - 1;
  return static_cast<int32_t>(span < max_seq_len ? span : max_seq_len);
}

struct AttnCall {
  int32_t dtype;
  const void* q;
  int32_t num_rows;
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t max_qlen;
  int32_t num_q_heads;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  const int32_t* block_table;
  int32_t max_blocks_per_seq;
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t window;
  float scale;
  int32_t partition_tokens;
  uint32_t flags;
  float* out;
  void* workspace;
  int64_t workspace_bytes;
  void* stream;
};

int32_t run_cross_attn(const AttnCall& c, const char* who) {
  using namespace yoco;
  if (c.dtype != YOCO_DTYPE_F32 && c.dtype != YOCO_DTYPE_BF16)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", who, c.dtype);
  if (c.num_seqs < 0 || c.num_rows < 0 || c.num_q_heads <= 0 || c.num_kv_heads <= 0 || c.num_blocks <= 0 ||
      c.max_blocks_per_seq <= 0 || c.max_seq_len < 0 || c.partition_tokens < 0 || c.workspace_bytes < 0 ||
      c.window < 0 || c.max_qlen < 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: negative or zero size argument", who);
  if (c.qsl == nullptr && (c.num_rows != c.num_seqs || c.max_qlen != 1))
    return fail(YOCO_ERR_INVALID_ARGUMENT,
                "%s: without query_start_loc there is one query row per request (num_rows %d, num_seqs %d, "
                "max_query_len %d)", who, c.num_rows, c.num_seqs, c.max_qlen);
  if (c.num_q_heads % c.num_kv_heads != 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who,
                c.num_q_heads, c.num_kv_heads);
  if ((c.flags & ~YOCO_FLAG_REVERSE_ORDER) != 0) return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: unknown flags", who);
  if (!std::isfinite(c.scale)) return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: scale is not finite", who);
  if (c.partition_tokens % 64 != 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: partition_tokens %d is not a multiple of 64", who,
                c.partition_tokens);
  if (c.k_scale != nullptr || c.v_scale != nullptr)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: cache scales are only read for an 8-bit cache", who);
  const int group = c.num_q_heads / c.num_kv_heads;
  if (!supported_dim(c.head_dim))
    return fail(YOCO_ERR_UNSUPPORTED, "%s: head_dim %d not in {64,128,256}", who, c.head_dim);
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: %d query heads per KV head not in {1,2,4,8}", who, group);
  if (!is_pow2(c.block_size) || c.block_size > 256)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: block_size %d is not a power of two <= 256", who, c.block_size);
  if (c.partition_tokens > max_partition(c.block_size))
    return fail(YOCO_ERR_UNSUPPORTED, "%s: partition_tokens %d exceeds %d for block_size %d", who,
                c.partition_tokens, max_partition(c.block_size), c.block_size);
  if (c.qsl != nullptr && c.num_seqs > kMaxQueueSeqs)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: %d requests with query_start_loc exceed %d", who, c.num_seqs,
                kMaxQueueSeqs);
  if (c.num_seqs == 0 || c.num_rows == 0 || c.max_qlen == 0) return YOCO_OK;
  if (c.q == nullptr || c.k_cache == nullptr || c.v_cache == nullptr || c.block_table == nullptr ||
      c.seq_lens == nullptr || c.out == nullptr)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: null pointer", who);
  if (!aligned16(c.q) || !aligned16(c.k_cache) || !aligned16(c.v_cache) || !aligned16(c.out))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: q, caches and out must be 16-byte aligned", who);

  const int32_t span = effective_len(c.max_seq_len, c.max_qlen, c.window);
  const int32_t part = resolve_partition(c.num_seqs, c.num_kv_heads, c.head_dim, span, c.block_size,
                                         c.partition_tokens);
  const int32_t nparts = num_partitions(span, part);
  if (nparts > kMaxParts)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: %d partitions per request exceed %d", who, nparts, kMaxParts);
  const int qpi = c.qsl == nullptr ? 0 : (c.max_qlen > 1 ? 8 / group : 1);
  const int64_t groups = qpi == 0 ? 1 : yoco::ceil_div(c.max_qlen, qpi);
  const int64_t items = static_cast<int64_t>(c.num_seqs) * c.num_kv_heads * groups * nparts;
  if (items > 0x7fffffffLL)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: %lld work items is too many", who, (long long)items);
  const WorkspaceLayout ws = workspace_layout(c.num_rows, c.num_q_heads, c.head_dim, nparts);
  if (c.workspace_bytes < ws.total)
    return fail(YOCO_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %lld bytes, need %lld", who,
                (long long)c.workspace_bytes, (long long)ws.total);
  if (c.workspace == nullptr || !aligned16(c.workspace))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "%s: workspace must be a 16-byte aligned pointer", who);
  const int64_t merge_grid = static_cast<int64_t>(c.num_seqs) * c.max_qlen * c.num_q_heads;
  if (nparts > 1 && merge_grid > 0x7fffffffLL)
    return fail(YOCO_ERR_UNSUPPORTED, "%s: merge grid of %lld workgroups is too many", who, (long long)merge_grid);

  AttnArgs a;
  a.q = c.q;
  a.k = c.k_cache;
  a.v = c.v_cache;
  a.block_table = c.block_table;
  a.seq_lens = c.seq_lens;
  a.out = c.out;
  char* wsb = static_cast<char*>(c.workspace);
  a.ws_acc = nparts > 1 ? reinterpret_cast<float*>(wsb + ws.acc_offset) : nullptr;
  a.ws_ml = nparts > 1 ? reinterpret_cast<float*>(wsb + ws.ml_offset) : nullptr;
  a.queue = c.num_seqs <= kMaxQueueSeqs ? reinterpret_cast<uint32_t*>(wsb) : nullptr;
  a.head_stride = c.block_size * c.head_dim;
  a.block_stride = static_cast<int64_t>(c.num_kv_heads) * c.block_size * c.head_dim;
  a.num_seqs = c.num_seqs;
  a.num_q_heads = c.num_q_heads;
  a.num_kv_heads = c.num_kv_heads;
  a.num_blocks = c.num_blocks;
  a.block_size = c.block_size;
  a.bs_shift = ilog2(c.block_size);
  a.max_blocks = c.max_blocks_per_seq;
  const int64_t cap = static_cast<int64_t>(c.max_blocks_per_seq) * c.block_size;
  a.len_cap = static_cast<int32_t>(cap < c.max_seq_len ? cap : c.max_seq_len);
  a.part_tokens = part;
  a.num_parts = nparts;
  a.scale_log2 = c.scale * kLog2e;
  a.flags = c.flags;
  a.qsl = c.qsl;
  a.num_rows = c.num_rows;
  a.max_qlen = c.max_qlen;
  a.window = c.window;

  hipStream_t s = static_cast<hipStream_t>(c.stream);
  clear_launch_error();
  const int launched = c.dtype == YOCO_DTYPE_BF16 ? dispatch_dim<true>(c.head_dim, group, qpi, a, items, s)
                                                  : dispatch_dim<false>(c.head_dim, group, qpi, a, items, s);
  if (launched == 0) return fail(YOCO_ERR_UNSUPPORTED, "%s: no kernel for this shape", who);
  if (launched < 0) return fail(YOCO_ERR_HIP, "%s: occupancy query failed on the current device", who);
  if (nparts > 1) {
    const uint32_t mgrid = static_cast<uint32_t>(merge_grid);
    switch (c.head_dim) {
      case 64: hipLaunchKernelGGL(cross_attn_merge_kernel<64>, dim3(mgrid), dim3(kThreads), 0, s, a); break;
      case 128: hipLaunchKernelGGL(cross_attn_merge_kernel<128>, dim3(mgrid), dim3(kThreads), 0, s, a); break;
      default: hipLaunchKernelGGL(cross_attn_merge_kernel<256>, dim3(mgrid), dim3(kThreads), 0, s, a); break;
    }
  }
  return launch_result(who);
}

}  // namespace

extern "C" int32_t yoco_cross_attn_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_seq_len, int32_t block_size,
                                                    int32_t partition_tokens) {
  if (partition_tokens < 0 || max_seq_len < 0 || block_size <= 0) return -1;
  return resolve_partition(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, partition_tokens);
}

extern "C" int64_t yoco_cross_attn_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t max_seq_len, int32_t block_size,
                                                  int32_t partition_tokens) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      block_size <= 0 || partition_tokens < 0)
    return -1;
  const int32_t p = resolve_partition(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, partition_tokens);
  return workspace_layout(num_seqs, num_q_heads, head_dim, num_partitions(max_seq_len, p)).total;
}

extern "C" int64_t yoco_cross_attn_varlen_workspace_size(int32_t num_rows, int32_t num_seqs, int32_t num_q_heads,
                                                         int32_t num_kv_heads, int32_t head_dim,
                                                         int32_t max_seq_len, int32_t max_query_len,
                                                         int32_t window, int32_t block_size,
                                                         int32_t partition_tokens) {
  if (num_rows < 0 || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      max_query_len < 0 || window < 0 || block_size <= 0 || partition_tokens < 0)
    return -1;
  const int32_t span = effective_len(max_seq_len, max_query_len, window);
  const int32_t p = resolve_partition(num_seqs, num_kv_heads, head_dim, span, block_size, partition_tokens);
  return workspace_layout(num_rows, num_q_heads, head_dim, num_partitions(span, p)).total;
}

extern "C" int32_t yoco_cross_attn(int32_t dtype, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                   const void* k_cache, const void* v_cache, int32_t num_blocks,
                                   int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                   int32_t partition_tokens, uint32_t flags, float* out, void* workspace,
                                   int64_t workspace_bytes, void* stream) {
  const AttnCall c{dtype, q, num_seqs, nullptr, num_seqs, 1, num_q_heads, k_cache, v_cache, nullptr, nullptr,
                   num_blocks, num_kv_heads, block_size, head_dim, block_table, max_blocks_per_seq, seq_lens,
                   max_seq_len, 0, scale, partition_tokens, flags, out, workspace, workspace_bytes, stream};
  return run_cross_attn(c, "cross_attn");
}

extern "C" int32_t yoco_cross_attn_varlen(int32_t dtype, const void* q, int32_t num_rows,
                                          const int32_t* query_start_loc, int32_t num_seqs, int32_t max_query_len,
                                          int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                          const float* k_scale, const float* v_scale, int32_t num_blocks,
                                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                                          const int32_t* block_table, int32_t max_blocks_per_seq,
                                          const int32_t* seq_lens, int32_t max_seq_len, int32_t window,
                                          float scale, int32_t partition_tokens, uint32_t flags, float* out,
                                          void* workspace, int64_t workspace_bytes, void* stream) {
  const AttnCall c{dtype, q, num_rows, query_start_loc, num_seqs, max_query_len, num_q_heads, k_cache, v_cache,
                   k_scale, v_scale, num_blocks, num_kv_heads, block_size, head_dim, block_table,
                   max_blocks_per_seq, seq_lens, max_seq_len, window, scale, partition_tokens, flags, out,
                   workspace, workspace_bytes, stream};
  return run_cross_attn(c, "cross_attn_varlen");
}
