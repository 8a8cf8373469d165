// Device code of yoco_cross_attn, shared by the translation units that
// instantiate it (one per cache element type, compiled in parallel) and by the
// host code in cross_attn.hip.  What the kernels compute and how is described
// at the top of cross_attn.hip.
#pragma once

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "yoco_internal.h"

namespace yoco_attn {


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

// How the key range of one context (m tokens) is cut into partitions.  The
// first big(m) partitions hold P tokens each ("big"); the rest -- at least
// min(m, T) and fewer than T + P tokens -- is cut into pieces of Ps tokens,
// the last one shorter ("small"; an empty range has one, empty, small
// partition).  T = 0 with Ps = P gives ceil(m/P) partitions of P tokens.
// The persistent schedule numbers every big item before every small one, so
// the work ends on short items.
struct Split {
  int32_t P;    // tokens of a full partition
  int32_t Ps;   // tokens of a tail piece (Ps <= P)
  int32_t T;    // tokens at the end of every range that go into pieces
  __host__ __device__ int big(int m) const { return m > T ? (m - T) / P : 0; }
  __host__ __device__ int small(int m) const {
    const int rest = m - big(m) * P;
    return m <= 0 ? 1 : rest / Ps + (rest % Ps != 0 ? 1 : 0);
  }
  __host__ __device__ int parts(int m) const { return big(m) + small(m); }
  // parts(m) == 1, without a division: T = 0 comes with Ps = P, and T > 0
  // is at least Ps unless every range is shorter than Ps.
  __host__ __device__ bool single(int m) const { return m <= Ps; }
  // First token (relative to the range's start) and length of partition
  // `part` of a range with nbig big partitions.
  __host__ __device__ int start(int nbig, int part) const {
    return part < nbig ? part * P : nbig * P + (part - nbig) * Ps;
  }
  __host__ __device__ int len(int nbig, int part) const { return part < nbig ? P : Ps; }
};

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
  Split split;          // partitions of each context's key range
  int32_t num_parts;    // partition slots per query row in the workspace (max over contexts)
  float scale_log2;     // scale * log2(e)
  uint32_t flags;
  const int32_t* qsl;   // query_start_loc [num_seqs+1] (several query rows per request), nullptr otherwise
  int32_t num_rows;     // query rows of q and out (num_seqs without qsl)
  int32_t max_qlen;     // query rows per request are clamped to this (1 without qsl)
  int32_t window;       // sliding window in tokens; 0 = the whole context
  const float* k_scale; // FP8 cache: [num_blocks][Hkv][bs] per-row scales, else nullptr
  const float* v_scale;
};

// First context position any query of a request can see: its queries sit at
// positions n-ql .. n-1, and with a window of W tokens the earliest key of the
// first one is n-ql-W+1 (without a window, position 0).
__host__ __device__ inline int range_lo(int n, int ql, int window) {
  if (window <= 0) return 0;
  const int lo = n - ql - window + 1;
  return lo > 0 ? lo : 0;
}

// Cache element types: fp32 (queries fp32), bf16 and FP8 E4M3 with per-row
// scales (queries bf16).
constexpr int kF32 = 0, kBF16 = 1, kFP8 = 2;
template <int kT> constexpr int kElemBytesOf = kT == kF32 ? 4 : (kT == kBF16 ? 2 : 1);
template <int kT> constexpr int kQBytesOf = kT == kF32 ? 4 : 2;

template <int kT, int D>
struct Layout {
  static constexpr int kEpc = 16 / kElemBytesOf<kT>;      // elements per 16-byte chunk
  static constexpr int kChunks = D / kEpc;                // chunks per row
  // lanes per row: two chunks per lane (fp32, bf16), one (FP8, whose rows are short)
  static constexpr int kLpr = kT == kFP8 ? (kChunks < 16 ? kChunks : 16) : (kChunks / 2 < 16 ? kChunks / 2 : 16);
  static constexpr int kCpl = kChunks / kLpr;             // chunks per lane
  static constexpr int kRpw = 64 / kLpr;                  // rows per wave instruction
  static constexpr int kU = kT == kFP8 ? 4 : 2;           // row sets per iteration (same bytes in flight)
  static constexpr int kIterTokens = kRpw * kU;
  static constexpr int kQpc = kEpc * kQBytesOf<kT> / 16;  // 16-byte query chunks per cache chunk
};

// Dot product of one 16-byte chunk of q with one of k, accumulated into acc.
template <int kT>
__device__ __forceinline__ float chunk_dot(const uint4& q, const uint4& k, float acc);

template <>
__device__ __forceinline__ float chunk_dot<kBF16>(const uint4& q, const uint4& k, float acc) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k.x), __builtin_bit_cast(bf2, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k.y), __builtin_bit_cast(bf2, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k.z), __builtin_bit_cast(bf2, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, k.w), __builtin_bit_cast(bf2, q.w), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<kF32>(const uint4& q, const uint4& k, float acc) {
  acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
  return acc;
}

// The elements of a 16-byte chunk as fp32 (exact widening).
template <int kT>
__device__ __forceinline__ void decode_chunk(const uint4& c, float (&x)[16 / kElemBytesOf<kT>]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  if constexpr (kT == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  } else if constexpr (kT == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);   // bytes 0, 1
      const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);    // bytes 2, 3
      x[4 * i] = lo.x;
      x[4 * i + 1] = lo.y;
      x[4 * i + 2] = hi.x;
      x[4 * i + 3] = hi.y;
    }
  }
}

// Sixteen FP8 E4M3 codes as sixteen bf16 values (exact: every E4M3 value is a
// bf16 value), packed in pairs in element order, for v_dot2_f32_bf16.
__device__ __forceinline__ void fp8_to_bf16(const uint4& c, uint4& lo8, uint4& hi8) {
#define YOCO_PAIR(w, hi) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((w), 1.0f, (hi)))
  lo8 = make_uint4(YOCO_PAIR(c.x, false), YOCO_PAIR(c.x, true), YOCO_PAIR(c.y, false), YOCO_PAIR(c.y, true));
  hi8 = make_uint4(YOCO_PAIR(c.z, false), YOCO_PAIR(c.z, true), YOCO_PAIR(c.w, false), YOCO_PAIR(c.w, true));
#undef YOCO_PAIR
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

// One step of a reduce-scatter across lane bit M of a wavefront (M = 4, 8,
// 16 or 32).  Every lane holds a, its value of the half that the lanes with
// the bit clear keep, and b, its value of the half that the lanes with the
// bit set keep; the result, in every lane, is the kept half's value from the
// lane of the pair with the bit clear (c) and from the one with the bit set
// (s).  M = 16, 32: one v_permlane16_swap / v_permlane32_swap (the swap moves
// exactly the two halves that change hands); M = 8: DPP rotation by 8 within
// each 16-lane row (= lane xor 8); M = 4: LDS swizzle with xor mask 4.
template <int M>
__device__ __forceinline__ void exchange_halves(float a, float b, float& c, float& s) {
  static_assert(M == 4 || M == 8 || M == 16 || M == 32, "lane bit 2 to 5");
  if constexpr (M == 16 || M == 32) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    u2 r;
    if constexpr (M == 16) {
      r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    } else {
      r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    }
    c = __uint_as_float(r.x);
    s = __uint_as_float(r.y);
  } else {
    const bool up = (threadIdx.x & M) != 0;
    const int send = __float_as_int(up ? a : b);
    int got;
    if constexpr (M == 8) {
      got = __builtin_amdgcn_update_dpp(0, send, 0x128, 0xf, 0xf, false);
    } else {
      got = __builtin_amdgcn_ds_swizzle(send, 0x101f);
    }
    const float recv = __int_as_float(got);
    c = up ? recv : a;
    s = up ? b : recv;
  }
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

// Merge the partials of one (query row, query head):
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// S workgroups per (request, query row of the request, head), each for D/S
// of head_dim (S > 1 when there are few such triples, so that the merge
// still spreads over the GPU); rows past the request's query count return at
// once.  256 threads: thread t owns float4 slice t % (D/4/S) of its part of
// head_dim and partitions p = t / (D/4/S) + k * (256 / (D/4/S)).  Each thread sums its partitions relative
// to its own running maximum in one pass (the loads of a batch of 8
// partitions are all in flight at once); the groups are then rescaled and
// added in group order through LDS (deterministic).  Rows whose context fits one partition were finished by
// the first kernel.
template <int D, int S>
__global__ __launch_bounds__(kThreads) void cross_attn_merge_kernel(AttnArgs a) {
  constexpr int kSlices = D / 4 / S;             // float4 slices of a head this workgroup merges
  constexpr int kGroups = kThreads / kSlices;    // partition groups
  __shared__ float4 s_num[kGroups][kSlices];
  __shared__ float s_den[kGroups];
  __shared__ float s_max[kGroups];
  const int64_t pair = blockIdx.x / S;           // (request, query row, head)
  const int part_of_d = static_cast<int>(blockIdx.x - pair * S);
  const int64_t per_req = static_cast<int64_t>(a.max_qlen) * a.num_q_heads;
  const int r = static_cast<int>(pair / per_req);
  const int rem = static_cast<int>(pair - r * per_req);
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
  const int m = n - range_lo(n, ql, a.window);
  if (a.split.single(m)) return;
  const int np = a.split.parts(m);
  const int64_t rh = static_cast<int64_t>(row) * a.num_q_heads + h;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + rh * a.num_parts;
  const float4* acc = reinterpret_cast<const float4*>(a.ws_acc + rh * a.num_parts * D) + part_of_d * kSlices;
  const int slice = tid % kSlices;
  const int grp = tid / kSlices;

  // One pass, online: each batch issues all of its loads before using any,
  // and the running sums are rescaled when a larger maximum comes in.
  constexpr int kBatch = 8;
  float m_loc = kInitMax;
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float den = 0.0f;
  for (int p0 = grp; p0 < np; p0 += kGroups * kBatch) {
    float2 part[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int p = p0 + k * kGroups;
      if (p < np) {
        part[k] = ml[p];
        v[k] = acc[static_cast<int64_t>(p) * (D / 4) + slice];
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (p0 + k * kGroups >= np) break;
      if (part[k].x > m_loc) {
        const float c = exp2f(m_loc - part[k].x);
        den *= c;
        num.x *= c;
        num.y *= c;
        num.z *= c;
        num.w *= c;
        m_loc = part[k].x;
      }
      const float w = exp2f(part[k].x - m_loc);
      den = fmaf(w, part[k].y, den);
      num.x = fmaf(w, v[k].x, num.x);
      num.y = fmaf(w, v[k].y, num.y);
      num.z = fmaf(w, v[k].z, num.z);
      num.w = fmaf(w, v[k].w, num.w);
    }
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
    reinterpret_cast<float4*>(a.out + rh * D)[part_of_d * kSlices + tid] =
        make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  }
}

template <int kT, int D>
struct RowSet {
  uint4 k[Layout<kT, D>::kU][Layout<kT, D>::kCpl];
  uint4 v[Layout<kT, D>::kU][Layout<kT, D>::kCpl];
  bool valid[Layout<kT, D>::kU];
  int pos[Layout<kT, D>::kU];        // logical position of the row (masks of the several-query path)
  float ks[Layout<kT, D>::kU];       // FP8: the row's K and V scales
  float vs[Layout<kT, D>::kU];
};

// Shared memory of one workgroup: block-table slices and queries of the
// current and the next work item (double buffered), the per-wavefront softmax
// states and, for the persistent schedule, every request's clamped length,
// (several-query path) its first query row, and the prefix of work-item
// counts.  VG = query vectors per item (G heads times the rows per item).
template <int kT, int D, int VG, bool kVar>
struct AttnSmem {
  static constexpr int kQChunks = VG * D * kQBytesOf<kT> / 16;     // 16-byte chunks of an item's queries
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

// `off` and `len`: the partition's first token relative to lo, and its
// length (the caller knows whether it is a full partition or a piece).
__device__ __forceinline__ Item make_item(bool valid, int r, int g, int part, int off, int len, int n, int lo,
                                          int row0, int nq, int pbase, int bs_shift) {
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
  it.start = it.lo + (valid ? uniform(off) : 0);
  it.end = min(it.start + (valid ? uniform(len) : 0), it.n);
  // An item without rows stages (harmlessly) the first table entry of its
  // row: its start may lie past the row's last entry.
  it.first_blk = it.end > it.start ? it.start >> bs_shift : 0;
  it.num_blk = it.end > it.start ? ((it.end - 1) >> bs_shift) - it.first_blk + 1 : 0;
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
template <int kT, int D, int G, int QPI>
__global__ __launch_bounds__(kThreads) void cross_attn_kernel(AttnArgs a) {
  using L = Layout<kT, D>;
  constexpr bool kVar = QPI > 0;
  constexpr bool kF8 = kT == kFP8;
  constexpr int kQ = kVar ? QPI : 1;                               // query rows per item
  constexpr int VG = G * kQ;                                       // query vectors per item
  using Smem = AttnSmem<kT, D, VG, kVar>;
  constexpr int kEpc = L::kEpc, kLpr = L::kLpr, kCpl = L::kCpl, kRpw = L::kRpw, kU = L::kU, kQpc = L::kQpc;
  constexpr int kIterTokens = L::kIterTokens;
  constexpr int kElemBytes = kElemBytesOf<kT>;                     // cache element bytes
  constexpr int kQBytes = kQBytesOf<kT>;                           // query element bytes
  constexpr int kQChunks = Smem::kQChunks;
  constexpr int kHeadChunks = D * kQBytes / 16;                    // 16-byte chunks of one query vector
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
      nb = a.split.big(m) * a.num_kv_heads * groups;
      ns = a.split.small(m) * a.num_kv_heads * groups;
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
    if (k >= total) return make_item(false, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, a.bs_shift);
    // The reverse order reverses the whole order when every context is cut
    // into full partitions only (T = 0), so a layer starts where the previous
    // one ended; with tail pieces it reverses the big items and, separately,
    // the small ones, so the pieces stay last.
    const bool k_big = k < total_big;
    const uint32_t kk = !reverse ? k
                        : a.split.T == 0 ? total - 1u - k
                        : (k_big ? total_big - 1u - k : total + total_big - 1u - k);
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
    // a full partition starts at sub * P; piece sub after the nbig full ones
    const int nbig = big ? 0 : a.split.big(n - lo);
    const int part = nbig + sub;
    const int off = big ? sub * a.split.P : nbig * a.split.P + sub * a.split.Ps;
    const int len = big ? a.split.P : a.split.Ps;
    if constexpr (kVar) {
      return make_item(true, r, g, part, off, len, n, lo, sm.qs[r] + qgrp * kQ, min(kQ, ql - qgrp * kQ),
                       n - ql + qgrp * kQ, a.bs_shift);
    } else {
      return make_item(true, r, g, part, off, len, n, lo, r, 1, n - 1, a.bs_shift);
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
            ((static_cast<int64_t>(qrow) * a.num_q_heads + it.g * G + (v - i * G)) * D) * kQBytes);
        st_q[j] = qg[c - v * kHeadChunks];
      }
    } else {
      const uint4* qg = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                       (static_cast<int64_t>(it.r) * a.num_q_heads + it.g * G) * D *
                                                           kQBytes);
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
  auto load = [&](RowSet<kT, D>& rs, const Item& it, int buf, int iter) {
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
      // slice entry of the row; a masked row reads entry 0 (its value is unused)
      const int blk = sm.blocks[buf][in_range ? (j >> a.bs_shift) - it.first_blk : 0];
      rs.valid[u] = in_range && blk >= 0;
      rs.pos[u] = j;
      const int64_t off = rs.valid[u] ? (static_cast<int64_t>(blk) * a.block_stride +
                                         static_cast<int64_t>(j & off_mask) * D) * kElemBytes
                                      : dummy_off;
#pragma unroll
      for (int i = 0; i < kCpl; ++i) {
        const int64_t c = off + static_cast<int64_t>((cl + kLpr * i) * kEpc) * kElemBytes;
        rs.k[u][i] = yoco::load_stream(kb + c);
        rs.v[u][i] = yoco::load_stream(vb + c);
      }
      if constexpr (kF8) {
        // the row's scales: element offset / D is the row index in [block][head][slot] order
        const int64_t sidx = off / D + static_cast<int64_t>(it.g) * a.block_size;
        rs.ks[u] = a.k_scale[sidx];
        rs.vs[u] = a.v_scale[sidx];
      }
    }
  };

  // Rows of one iteration of a wavefront: iteration `iter` of item `it`
  // (slice in LDS buffer `buf`), or, once iter reaches num_iters, the
  // wavefront's first rows of item `nx` (block ids from the staging
  // registers).  One branch-free set of loads either way.
  auto load_step = [&](RowSet<kT, D>& rs, const Item& it, int buf, int iter, int num_iters, const Item& nx) {
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
      // slice entry of the row in the current item; rows of the next item, and
      // masked rows, read entry 0 instead (unused: an item without rows has
      // first_blk 0 while its start may lie far past the slice)
      const int lds_blk = sm.blocks[buf][in_range && !to_nx ? (j >> a.bs_shift) - it.first_blk : 0];
      const int blk = to_nx ? st_nb[u] : lds_blk;
      rs.valid[u] = in_range && blk >= 0;
      rs.pos[u] = j;
      const int64_t off = rs.valid[u] ? (static_cast<int64_t>(blk) * a.block_stride +
                                         static_cast<int64_t>(j & off_mask) * D) * kElemBytes
                                      : dummy_off;
#pragma unroll
      for (int i = 0; i < kCpl; ++i) {
        const int64_t c = off + static_cast<int64_t>((cl + kLpr * i) * kEpc) * kElemBytes;
        rs.k[u][i] = yoco::load_stream(kb + c);
        rs.v[u][i] = yoco::load_stream(vb + c);
      }
      if constexpr (kF8) {
        // the row's scales: element offset / D is the row index in [block][head][slot] order
        const int64_t sidx = off / D + static_cast<int64_t>(g) * a.block_size;
        rs.ks[u] = a.k_scale[sidx];
        rs.vs[u] = a.v_scale[sidx];
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

  auto compute = [&](const RowSet<kT, D>& rs, int buf) {
    // FP8: every K chunk is widened once to bf16 pairs, for all heads.
    constexpr int kKw = kF8 ? 2 : 1;
    uint4 kw[kU][kCpl][kKw];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < kCpl; ++i) {
        if constexpr (kF8) {
          fp8_to_bf16(rs.k[u][i], kw[u][i][0], kw[u][i][1]);
        } else {
          kw[u][i][0] = rs.k[u][i];
        }
      }
    constexpr int kDotT = kF8 ? kBF16 : kT;
    float s[kU][VG];
#pragma unroll
    for (int h = 0; h < VG; ++h) {
      uint4 qh[kCpl][kQpc];
#pragma unroll
      for (int i = 0; i < kCpl; ++i)
#pragma unroll
        for (int c = 0; c < kQpc; ++c) qh[i][c] = sm.q[buf][(h * D + (cl + kLpr * i) * kEpc) * kQBytes / 16 + c];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float t = 0.0f;
#pragma unroll
        for (int i = 0; i < kCpl; ++i)
#pragma unroll
          for (int c = 0; c < kQpc; ++c) t = chunk_dot<kDotT>(qh[i][c], kw[u][i][c], t);
        t = group_sum<kLpr>(t);
        bool ok = rs.valid[u];
        if constexpr (kVar) {
          const int qi = h / G;
          ok = ok && rs.pos[u] >= qlo[qi] && rs.pos[u] < qhi[qi];
        }
        const float sc = kF8 ? a.scale_log2 * rs.ks[u] : a.scale_log2;
        s[u][h] = ok ? t * sc : -INFINITY;
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
        // FP8: the row's V scale joins the weight (zero for a masked row,
        // whose scale may be anything).
        if constexpr (kF8) p[h] *= rs.valid[u] ? rs.vs[u] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < kCpl; ++i) {
        // A masked row (p = 0) read some other row, which may hold NaN:
        // zero its values so that it adds exactly nothing.
        const uint4 vc = rs.valid[u] ? rs.v[u][i] : make_uint4(0u, 0u, 0u, 0u);
        float x[kEpc];
        decode_chunk<kT>(vc, x);
#pragma unroll
        for (int e = 0; e < kEpc; ++e) {
#pragma unroll
          for (int h = 0; h < VG; ++h) acc[h][i][e] = fmaf(p[h], x[e], acc[h][i][e]);
        }
      }
    }
  };

  // The first item (workgroup w starts with item w; the persistent schedule
  // fetches the next one while it runs).
  Item cur, nxt;
  // with a workgroup for every item (the grid is at most the item count) no
  // fetch can return an item: none is made
  const bool grid_covers = persistent && gridDim.x >= total;
  bool nxt_known = !persistent || grid_covers;
  if (persistent) {
    cur = item_at(blockIdx.x);
    nxt = grid_covers ? make_item(false, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, a.bs_shift) : cur;
  } else {
    const uint32_t items = static_cast<uint32_t>(R) * a.num_kv_heads * a.num_parts;
    const uint32_t item = reverse ? items - 1u - blockIdx.x : blockIdx.x;
    const uint32_t pairs = static_cast<uint32_t>(R) * a.num_kv_heads;
    const int part = static_cast<int>(item / pairs);
    const uint32_t rg = item % pairs;
    const int r = static_cast<int>(rg / a.num_kv_heads);
    int n = a.seq_lens[r];
    n = n < 0 ? 0 : (n > a.len_cap ? a.len_cap : n);
    const int lo = range_lo(n, 1, a.window);
    const int nbig = a.split.big(n - lo);
    cur = make_item(true, r, static_cast<int>(rg % a.num_kv_heads), part, a.split.start(nbig, part),
                    a.split.len(nbig, part), n, lo, r, 1, n - 1, a.bs_shift);
    nxt = make_item(false, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, a.bs_shift);
  }

  RowSet<kT, D> buf_a, buf_b;
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

      // Combine the row groups of the wavefront (lanes with the same cl) by
      // a reduce-scatter over the lane's row bits, widest first: at each step
      // the two lanes of a pair keep one half of their values each and take
      // the partner's copy of that half, so every value is combined by one
      // lane only; (m, l) are combined in both lanes of the pair, in the same
      // operand order.  A lane ends with kNV * kLpr / 64 = D / 64 consecutive
      // values (first value index `keep`) of every query vector.
      constexpr int kNV = kCpl * kEpc;
      constexpr int kKeep = kNV * kLpr / 64;
      static_assert(kKeep >= 1 && kEpc % kKeep == 0, "kept values lie in one chunk");
      int keep = 0;
      auto combine_step = [&](auto mask_c, auto cur_c) {
        constexpr int M = decltype(mask_c)::value;
        constexpr int kHalf = decltype(cur_c)::value / 2;
        keep += (lane & M) != 0 ? kHalf : 0;
#pragma unroll
        for (int h = 0; h < VG; ++h) {
          float mc, ms, lc, ls;
          exchange_halves<M>(m[h], m[h], mc, ms);
          exchange_halves<M>(lsum[h], lsum[h], lc, ls);
          const float mx = fmaxf(mc, ms);
          const float fc = exp2f(mc - mx);
          const float fs = exp2f(ms - mx);
          lsum[h] = lc * fc + ls * fs;
          m[h] = mx;
#pragma unroll
          for (int j = 0; j < kHalf; ++j) {
            float c, t;
            exchange_halves<M>(acc[h][j / kEpc][j % kEpc], acc[h][(j + kHalf) / kEpc][(j + kHalf) % kEpc], c, t);
            acc[h][j / kEpc][j % kEpc] = c * fc + t * fs;
          }
        }
      };
      combine_step(std::integral_constant<int, 32>(), std::integral_constant<int, kNV>());
      if constexpr (kLpr <= 16) combine_step(std::integral_constant<int, 16>(), std::integral_constant<int, kNV / 2>());
      if constexpr (kLpr <= 8) combine_step(std::integral_constant<int, 8>(), std::integral_constant<int, kNV / 4>());
      if constexpr (kLpr <= 4) combine_step(std::integral_constant<int, 4>(), std::integral_constant<int, kNV / 8>());
      const int col0 = (cl + kLpr * (keep / kEpc)) * kEpc + keep % kEpc;
#pragma unroll
      for (int h = 0; h < VG; ++h) {
#pragma unroll
        for (int j = 0; j < kKeep; ++j) sm.acc[wave][h][col0 + j] = acc[h][0][j];
        if (lane == 0) {
          sm.ml[wave][h][0] = m[h];
          sm.ml[wave][h][1] = lsum[h];
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
      const bool whole = a.split.single(cur.n - cur.lo);
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
        if (whole) {
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


}  // namespace yoco_attn

#include "cross_attn_mfma.h"

namespace yoco_attn {

// ---- launch helpers (host) ------------------------------------------------------

// Workgroups of `kernel` resident on the current device at once (compute
// units x workgroups per compute unit), cached per device and kernel
// (defined in cross_attn.hip).
int resident_workgroups(const void* kernel, int per_cu_query(int*));

template <int kT, int D, int G, int QPI>
int per_cu_workgroups(int* out) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, cross_attn_kernel<kT, D, G, QPI>, kThreads, 0) ==
                 hipSuccess ? 0 : 1;
}

// Launch the attention kernel: persistent (grid = resident workgroups, at
// most one per work item) when the requests fit the LDS prefix, else one
// workgroup per work item.  Returns false if the occupancy query failed.
template <int kT, int D, int G, int QPI>
bool launch(AttnArgs a, int64_t items, hipStream_t stream) {
  int64_t grid = items;
  if (a.queue != nullptr) {
    const int slots = resident_workgroups(reinterpret_cast<const void*>(cross_attn_kernel<kT, D, G, QPI>),
                                          per_cu_workgroups<kT, D, G, QPI>);
    if (slots <= 0) return false;
    grid = items < slots ? items : slots;
  }
  hipLaunchKernelGGL((cross_attn_kernel<kT, D, G, QPI>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                     stream, a);
  return true;
}

// Query rows per work item: 0 for the decode kernel (one row per request);
// with query_start_loc, 8/G rows (eight query vectors per item) when a request
// may have more than one row, else 1.
template <int kT, int D, int G>
int dispatch_rows(int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  constexpr int kWide = 8 / G;
  if (qpi == 0) return launch<kT, D, G, 0>(a, items, stream) ? 1 : -1;
  if (qpi == 1) return launch<kT, D, G, 1>(a, items, stream) ? 1 : -1;
  if constexpr (kWide > 1) {
    if (qpi == kWide) return launch<kT, D, G, kWide>(a, items, stream) ? 1 : -1;
  }
  return 0;
}

template <int kT, int D>
int dispatch_group(int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  switch (group) {
    case 1: return dispatch_rows<kT, D, 1>(qpi, a, items, stream);
    case 2: return dispatch_rows<kT, D, 2>(qpi, a, items, stream);
    case 4: return dispatch_rows<kT, D, 4>(qpi, a, items, stream);
    case 8: return dispatch_rows<kT, D, 8>(qpi, a, items, stream);
    default: return 0;
  }
}

// 1: launched, 0: no kernel for the shape, -1: the occupancy query failed.
template <int kT>
int dispatch_dim(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  switch (head_dim) {
    case 64: return dispatch_group<kT, 64>(group, qpi, a, items, stream);
    case 128: return dispatch_group<kT, 128>(group, qpi, a, items, stream);
    case 256: return dispatch_group<kT, 256>(group, qpi, a, items, stream);
    default: return 0;
  }
}


// The matrix-core kernel (persistent schedule only): grid = resident
// workgroups, at most one per work item.
template <int kT, int D, int G, int QPI>
int per_cu_workgroups_mfma(int* out) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, cross_attn_mfma_kernel<kT, D, G, QPI>, kThreads, 0) ==
                 hipSuccess ? 0 : 1;
}

template <int kT, int D, int G, int QPI>
bool launch_mfma(AttnArgs a, int64_t items, hipStream_t stream) {
  const int slots = resident_workgroups(reinterpret_cast<const void*>(cross_attn_mfma_kernel<kT, D, G, QPI>),
                                        per_cu_workgroups_mfma<kT, D, G, QPI>);
  if (slots <= 0) return false;
  const int64_t grid = items < slots ? items : slots;
  hipLaunchKernelGGL((cross_attn_mfma_kernel<kT, D, G, QPI>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                     stream, a);
  return true;
}

// Query rows per item of the matrix-core kernel: 0 (decode), 1, or 16/G.
template <int kT, int D, int G>
int dispatch_rows_mfma(int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  constexpr int kWide = 16 / G;
  if (qpi == 0) return launch_mfma<kT, D, G, 0>(a, items, stream) ? 1 : -1;
  if (qpi == 1) return launch_mfma<kT, D, G, 1>(a, items, stream) ? 1 : -1;
  if (qpi == kWide) return launch_mfma<kT, D, G, kWide>(a, items, stream) ? 1 : -1;
  return 0;
}

template <int kT>
int dispatch_dim_mfma(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream) {
  auto by_group = [&](auto dim) -> int {
    constexpr int D = decltype(dim)::value;
    switch (group) {
      case 1: return dispatch_rows_mfma<kT, D, 1>(qpi, a, items, stream);
      case 2: return dispatch_rows_mfma<kT, D, 2>(qpi, a, items, stream);
      case 4: return dispatch_rows_mfma<kT, D, 4>(qpi, a, items, stream);
      case 8: return dispatch_rows_mfma<kT, D, 8>(qpi, a, items, stream);
      default: return 0;
    }
  };
  switch (head_dim) {
    case 64: return by_group(std::integral_constant<int, 64>());
    case 128: return by_group(std::integral_constant<int, 128>());
    case 256: return by_group(std::integral_constant<int, 256>());
    default: return 0;
  }
}

// Per element type (cross_attn_f32.hip, cross_attn_bf16.hip, cross_attn_fp8.hip;
// the matrix-core kernels in cross_attn_mfma_bf16.hip, cross_attn_mfma_fp8.hip):
// 1 = launched, 0 = no kernel for the shape, -1 = the occupancy query failed.
int dispatch_f32(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream);
int dispatch_bf16(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream);
int dispatch_fp8(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream);
int dispatch_mfma_bf16(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream);
int dispatch_mfma_fp8(int head_dim, int group, int qpi, const AttnArgs& a, int64_t items, hipStream_t stream);

}  // namespace yoco_attn
