// yoco_gated_retention: the self-decoder's gated retention, chunkwise, on the
// matrix cores.
//
// "YOCO_论文与推理数据流详解" §4.1-4.2: gated retention is a linear recurrence
// with an input-dependent forget gate gamma_t over a fixed-size state S per
// head (the current token's k_t^T v_t written in, the query reading q_t S),
// and the parallel, recurrent and chunkwise forms compute the same result;
// prefill uses the chunkwise form (matrix products inside a chunk, one state
// update per chunk boundary), decode the recurrent one.  The page's formulas
// did not survive; the library computes, per head,
//     S_t = gamma_t S_{t-1} + k_t^T v_t,     o_t = q_t S_t.
//
// Chunkwise form used here.  For a chunk of n <= 32 tokens starting from the
// state S (b_t = sum_{u<=t} log2 gamma_u inside the chunk):
//     o_t    = 2^{b_t} q_t S + sum_{s<=t} 2^{b_t - b_s} (q_t . k_s) v_s
//     S_next = 2^{b_{n-1}} S + sum_s 2^{b_{n-1} - b_s} k_s^T v_s
// which is the recurrence unrolled over the chunk (a one-row request inside
// a mixed batch is the case n = 1).
//
// A workgroup walks a run of a request's rows chunk by chunk for one head,
// with the head's fp32 state resident in registers (wavefront w owns value
// columns [w D/4, (w+1) D/4) for all key rows, in the MFMA accumulator
// layout).  Short requests are one run.  A long prefill is cut into segments
// of kSegRows rows that run in parallel, in two launches: the first computes,
// for every segment but the last, its contribution to the state from zero
// (the first segment from the stored state) and its total decay; the second
// starts each segment from the fold of the earlier segments' results
// (S_in(j) = G_{j-1} S_in(j-1) + dS_{j-1}, the recurrence being linear in the
// state) and produces the outputs, the last segment the final state.  Per
// chunk:
//   stage    Q, K, V rows (bf16) in LDS row-major, and K~ = w_s k_s split
//            into bf16 high and low parts, row-major too: the MFMA operands
//            that need them transposed (V^T, K~^T) come from transposed LDS
//            reads (ds_read_b64_tr_b16); the per-token decay terms are
//            computed a chunk ahead by one wavefront's prefix sum;
//   A = QK^T three 16x16 causal tiles (v_mfma_f32_16x16x32_bf16), each
//            scaled by 2^{b_t - b_s}, stored as bf16 high + low parts;
//   O        Q S (the state split into bf16 high + low in registers), rows
//            scaled by 2^{b_t}, plus A V;
//   S        2^{b_{n-1}} S + K~^T V; the state's own decay is kept in a
//            running scale while that stays above 2^-60 (the new keys are
//            weighted by its inverse instead), so the state is multiplied
//            out only when the scale would get too small.
// The next chunk's rows are loaded into registers while the current one is
// computed.  q, k and v are exact bf16 operands; every fp32 operand (state,
// A, K~) enters as two bf16 parts (~17 significant bits); sums are fp32.
// log2 gamma is clamped at -64, so a zero gate weighs 2^-64 instead of 0.
//
// Decode batches (at most one row per request) take the recurrent form
// instead: one workgroup per (request, head, 32-column slice of the state)
// streams its slice through registers with 16-byte loads and stores,
// S = gamma S + k^T v then o = q S, the partial products reduced over row
// groups in LDS.

#include <type_traits>

#include "yoco_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kC = 32;                  // tokens per chunk
constexpr int kRowPad = 8;              // bf16 elements of padding per LDS row
constexpr int kTrPad = 16;              // padding of the tiles read transposed
constexpr float kMinLog2Gate = -64.0f;
constexpr float kMinLazyScale = 0x1p-60f;   // smallest state scale kept apart from the state
constexpr int kSegRows = 2048;          // rows per segment of a long request (a multiple of kC)
constexpr int kMaxSegReqs = 2048;       // requests a segmented launch can schedule

// what a launch of the chunk kernel does
constexpr int kWhole = 0;               // each request in one run, from and back to its slot
constexpr int kSegState = 1;            // segments but the last: state contribution and decay only
constexpr int kSegFull = 2;             // every segment: outputs from the folded state; last: final state

struct RetArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* gamma;
  const int32_t* cu;
  const int32_t* slots;
  float* state;
  float* out;
  float* ws_state;                      // [segments][H][D][D] (segmented launches)
  float* ws_gate;                       // [segments][H]
  int32_t num_tokens;
  int32_t num_heads;
  int32_t num_slots;
  int32_t num_reqs;
};

template <int D>
struct RowTiles {
  uint16_t q[kC][D + kRowPad];          // row-major chunk rows (read by rows)
  uint16_t k[kC][D + kRowPad];
};

template <int D>
struct __attribute__((aligned(16))) RetSmem {
  union __attribute__((aligned(16))) {
    RowTiles<D> r;
    int32_t pref[kMaxSegReqs + 1];      // segment schedule, before the first chunk
  } u;
  // row-major tiles read through transposed LDS reads; a row stride of 8
  // banks mod 32 keeps the four rows of one read on disjoint banks
  uint16_t v[kC][D + kTrPad];           // V
  uint16_t kh[kC][D + kTrPad];          // K~ = w_s k_s (over the state scale), bf16 high part
  uint16_t kl[kC][D + kTrPad];          // low part
  uint16_t ah[kC][kC + kRowPad];        // decayed causal Q K^T, high part
  uint16_t al[kC][kC + kRowPad];        // low part
  float b[2][kC];                       // inclusive prefix of log2 gamma (by chunk parity)
  float g[2][kC];                       // 2^{b_t}
  float w[2][kC];                       // 2^{b_{n-1} - b_s}
};

__device__ __forceinline__ uint16_t bf16_bits(__bf16 h) { return __builtin_bit_cast(uint16_t, h); }

// x = hi + lo with hi, lo bf16 (hi the nearest bf16 to x).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

typedef short v4s __attribute__((ext_vector_type(4)));

// MFMA operand for k-slots 8gi .. 8gi+7 = rows r0 + 8gi + 0..7 of a row-major
// bf16 tile, for lane l16 of each 16-lane group: column c0 + l16.  Two
// transposed reads (ds_read_b64_tr_b16): in each 16-lane group lane i's slot
// j is element i % 4 of the 8 bytes lane 4j + i/4 addressed, so lane m
// addresses row r0 + 8gi + 4h + m/4, columns c0 + 4(m % 4) .. +3.
template <int kStride>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int r0, int c0, int gi, int l16) {
  const uint16_t* p0 = tile + (r0 + 8 * gi + (l16 >> 2)) * kStride + c0 + 4 * (l16 & 3);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)(p0));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)(p0 + 4 * kStride));
  const uint2 a = __builtin_bit_cast(uint2, lo);
  const uint2 b = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// Two values at once: hi = the nearest bf16 pair (packed, x0 in the low
// half), lo = the bf16 pair nearest to the remainders x - hi.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = yoco::pack_bf16x2(x0, x1);
  lo = yoco::pack_bf16x2(x0 - yoco::bf16_lo(hi), x1 - yoco::bf16_hi(hi));
}

// Rows [start, end) of request r after clamping its offsets to [0, num_tokens].
__device__ __forceinline__ void request_rows(const RetArgs& a, int r, int& start, int& end) {
  start = min(max(a.cu[r], 0), a.num_tokens);
  end = min(max(a.cu[r + 1], start), a.num_tokens);
}

// Segments of a request of `rows` rows; a request without rows has one,
// empty, segment, so every request has exactly one last segment.
__device__ __forceinline__ int num_segments(int rows) { return rows > 0 ? (rows + kSegRows - 1) / kSegRows : 1; }

// pref[r] = number of segments other than the last of requests 0..r-1
// (pref[R] = their total), in LDS.  Request r's segments are numbered
// pref[r] + r .. pref[r] + r + nseg - 1 in the workspace.
__device__ void segment_prefix(const RetArgs& a, int32_t* pref) {
  __shared__ int32_t wsum[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int R = a.num_reqs;
  const int per = (R + kThreads - 1) / kThreads;
  const int lo = min(tid * per, R);
  const int hi = min(lo + per, R);
  auto segs = [&](int r) {
    int b, e;
    request_rows(a, r, b, e);
    return num_segments(e - b) - 1;
  };
  int local = 0;
  for (int r = lo; r < hi; ++r) local += segs(r);
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  for (int r = lo; r < hi; ++r) {
    pref[r] = run;
    run += segs(r);
  }
  if (tid == kThreads - 1) pref[R] = run;
  __syncthreads();
}

// The request whose segments other than the last hold index seg: largest r
// with pref[r] <= seg (seg < pref[R]).
__device__ __forceinline__ int segment_owner(const int32_t* pref, int R, int seg) {
  int lo = 0, hi = R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= seg) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int D, int kMode>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gated_retention_kernel(RetArgs a) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr bool kOut = kMode != kSegState;   // this launch produces outputs
  constexpr int kCW = D / kWaves;             // value columns per wavefront
  constexpr int kCT = kCW / 16;               // 16-column tiles per wavefront
  constexpr int kDT = D / 16;                 // 16-row tiles of the state (key rows)
  constexpr int kKS = D / 32;                 // MFMA k-steps over head_dim
  constexpr int kRowChunks = D / 8;           // 16-byte chunks per row
  constexpr int kLoads = kC * kRowChunks / kThreads;   // row chunks per thread per matrix
  static_assert(kLoads >= 1 && kC * kRowChunks % kThreads == 0, "row staging split");
  static_assert(sizeof(RowTiles<D>) >= sizeof(int32_t) * (kMaxSegReqs + 1), "schedule fits the row tiles");
  static_assert(kSegRows % kC == 0, "segments hold whole chunks");
  using Smem = RetSmem<D>;
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int gi = lane >> 4;
  const int H = a.num_heads;
  const int item = blockIdx.x / H;
  const int h = blockIdx.x - item * H;

  // ---- this workgroup's run of rows [start, end) and where its state starts
  int r, start, end, seg = 0, j = 0, nseg = 1;
  if constexpr (kMode == kWhole) {
    r = item;
    request_rows(a, r, start, end);
  } else {
    segment_prefix(a, sm.u.pref);
    // Workgroups take every request's segments other than the last (whole
    // kSegRows-row runs) first, then the last segment of each request (the
    // short ones, and one-row decodes), so the launch ends on short work.
    // The workspace holds gridDim.x / H segments, enough whenever the offsets
    // are non-decreasing; overlapping requests could need more: then nothing
    // is computed rather than anything written past the workspace.
    const int inner = sm.u.pref[a.num_reqs];
    const int total = inner + a.num_reqs;
    if (item >= total || total > static_cast<int>(gridDim.x / H)) return;
    r = item < inner ? segment_owner(sm.u.pref, a.num_reqs, item) : item - inner;
    int rb, re;
    request_rows(a, r, rb, re);
    nseg = num_segments(re - rb);
    j = item < inner ? item - sm.u.pref[r] : nseg - 1;
    seg = sm.u.pref[r] + r + j;
    if (kMode == kSegState && j == nseg - 1) return;   // the last segment's contribution is not needed
    start = rb + j * kSegRows;
    end = min(start + kSegRows, re);
    __syncthreads();                                     // the schedule's LDS becomes row tiles
  }
  if (end <= start) return;                              // no rows: the state is left as it is
  const int slot = a.slots[r];
  const bool has_slot = slot >= 0 && slot < a.num_slots;
  const int cw = wave * kCW;
  const int64_t hs = static_cast<int64_t>(D) * D;       // floats per head state

  // ---- the state: S[16dt + 4gi + e][cw + 16ct + l16] in sacc[dt][ct][e]
  f32x4 sacc[kDT][kCT];
  auto load_state = [&](const float* src) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[dt][ct][e] = src[(16 * dt + 4 * gi + e) * D + cw + 16 * ct + l16];
  };
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(16 * dt + 4 * gi + e) * D + cw + 16 * ct + l16] = sacc[dt][ct][e];
  };
  auto zero_state = [&]() {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) sacc[dt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  };
  float* const slot_state = has_slot ? a.state + (static_cast<int64_t>(slot) * H + h) * hs : nullptr;
  auto ws_state = [&](int g) { return a.ws_state + (static_cast<int64_t>(g) * H + h) * hs; };
  if constexpr (kMode == kWhole) {
    if (has_slot) load_state(slot_state); else zero_state();
  } else if constexpr (kMode == kSegState) {
    // segment 0 starts from the stored state (and leaves a copy of it in the
    // last segment's entry, which the second launch reads instead of the slot
    // that the last segment overwrites); later segments start from zero
    if (j == 0 && has_slot) {
      load_state(slot_state);
      store_state(ws_state(seg + nseg - 1));
    } else {
      zero_state();
    }
  } else {
    const int first = seg - j;
    if (j == 0) {
      if (!has_slot) zero_state();
      else load_state(nseg > 1 ? ws_state(first + nseg - 1) : slot_state);
    } else {
      load_state(ws_state(first));                       // the state after segment 0
      for (int i = 1; i < j; ++i) {
        const float g = a.ws_gate[static_cast<int64_t>(first + i) * H + h];
        const float* d = ws_state(first + i);
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sacc[dt][ct][e] = g * sacc[dt][ct][e] + d[(16 * dt + 4 * gi + e) * D + cw + 16 * ct + l16];
      }
    }
  }

  // the strictly upper tile of A is never written by the chunk loop
  if constexpr (kOut) {
    for (int i = tid; i < 16 * 16; i += kThreads) {
      sm.ah[i >> 4][16 + (i & 15)] = 0;
      sm.al[i >> 4][16 + (i & 15)] = 0;
    }
  }

  // ---- chunk rows in registers: thread chunk c = tid + 256 i covers row
  // c / kRowChunks, elements 8 (c % kRowChunks) .. +7
  uint4 rq[kLoads], rk[kLoads], rv[kLoads];
  // a chunk's rows from a uniform 64-bit base plus 32-bit lane offsets
  // (H * D < 2^26, checked on the host, so 32 rows fit in 31 bits)
  const int row_elems = H * D;
  auto load_chunk = [&](int pos) {
    const int n = min(kC, end - pos);
    const int64_t base = static_cast<int64_t>(pos) * row_elems + h * D;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i;
      const int s = c / kRowChunks;
      const int cc = c - s * kRowChunks;
      // (the loads sit in their own branch: written as selects, the compiler
      // waits for them right away and the prefetch is lost)
      const int off = s * row_elems + 8 * cc;
      if (s < n) {
        if constexpr (kOut) rq[i] = yoco::load_stream(a.q + base + off);
        rk[i] = yoco::load_stream(a.k + base + off);
        rv[i] = yoco::load_stream(a.v + base + off);
      } else {
        rq[i] = rk[i] = rv[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  // ---- the decay terms of a chunk, by the last wavefront (idle while the
  // others compute the score tiles), one chunk ahead: lane t < n holds the
  // gate of row t; the chunk's gates are loaded two chunks ahead.
  float rg = 1.0f;
  auto load_gates = [&](int pos) {
    if (pos < end && lane < min(kC, end - pos)) rg = a.gamma[static_cast<int64_t>(pos) * H + h + lane * H];
  };
  auto decay_terms = [&](int pos, int buf) {
    const int n = min(kC, end - pos);
    float lg = lane < n ? fmaxf(__builtin_amdgcn_logf(rg), kMinLog2Gate) : 0.0f;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const float t = __shfl_up(lg, off, 64);
      if ((lane & 31) >= off) lg += t;
    }
    const float blast = __shfl(lg, n - 1, 64);
    if (lane < kC) {
      sm.b[buf][lane] = lg;
      sm.g[buf][lane] = __builtin_amdgcn_exp2f(lg);
      sm.w[buf][lane] = lane < n ? __builtin_amdgcn_exp2f(blast - lg) : 0.0f;
    }
  };
  if (wave == kWaves - 1) {
    load_gates(start);
    decay_terms(start, 0);
    load_gates(start + kC);
  }

  float gseg = 1.0f;                          // product of the chunks' total decays
  float scale = 1.0f;                         // the state is scale * sacc
  load_chunk(start);
  __syncthreads();                            // the first chunk's decay terms
  int buf = 0;
  for (int pos = start; pos < end; pos += kC, buf ^= 1) {
    const int n = min(kC, end - pos);
    // ---- the state's decay this chunk.  The registers hold S / scale: while
    // scale * 2^{b_{n-1}} stays above 2^-60 only the scale takes the decay
    // and the new keys are weighted by 1 / (scale 2^{b_{n-1}}) instead, which
    // saves multiplying the whole state every chunk; otherwise the state is
    // multiplied out and the scale returns to 1.
    const float glast = sm.g[buf][n - 1];
    const float cg = scale * glast;
    const bool lazy = cg >= kMinLazyScale;
    const float wscale = lazy ? 1.0f / cg : 1.0f;

    // ---- stage the rows: q and k (read by rows), v, and K~ = (w_s / ...) k
    // split into bf16 high and low parts, all row-major
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i;
      const int s = c / kRowChunks;
      const int cc = c - s * kRowChunks;
      if constexpr (kOut) {
        *reinterpret_cast<uint4*>(&sm.u.r.q[s][8 * cc]) = rq[i];
        *reinterpret_cast<uint4*>(&sm.u.r.k[s][8 * cc]) = rk[i];
      }
      *reinterpret_cast<uint4*>(&sm.v[s][8 * cc]) = rv[i];
      const float ws = sm.w[buf][s] * wscale;
      const uint32_t kw[4] = {rk[i].x, rk[i].y, rk[i].z, rk[i].w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        split2(ws * yoco::bf16_lo(kw[jj]), ws * yoco::bf16_hi(kw[jj]), hi[jj], lo[jj]);
      *reinterpret_cast<uint4*>(&sm.kh[s][8 * cc]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(&sm.kl[s][8 * cc]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    // the next chunk's rows travel while this one is computed
    if (pos + kC < end) load_chunk(pos + kC);
    __syncthreads();
    // ---- the next chunk's decay terms (and the gates after it)
    if (wave == kWaves - 1 && pos + kC < end) {
      decay_terms(pos + kC, buf ^ 1);
      load_gates(pos + 2 * kC);
    }
    // ---- A = Q K^T, causal tiles (t-tile, s-tile) = (0,0), (1,0), (1,1)
    if (kOut && wave < 3) {
      const int tt = (wave + 1) >> 1;
      const int ts = wave >> 1;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&sm.u.r.q[16 * tt + l16][32 * ks + 8 * gi]);
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&sm.u.r.k[16 * ts + l16][32 * ks + 8 * gi]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kb, acc, 0, 0, 0);
      }
      const int s = 16 * ts + l16;
      const float bs = sm.b[buf][s];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tt + 4 * gi + e;
        const float val = (s <= t && t < n) ? acc[e] * __builtin_amdgcn_exp2f(sm.b[buf][t] - bs) : 0.0f;
        __bf16 vh, vl;
        split_bf16(val, vh, vl);
        sm.ah[t][s] = bf16_bits(vh);
        sm.al[t][s] = bf16_bits(vl);
      }
    }
    // the score tiles are read below; the state pass writes none (its next
    // chunk's decay terms go to the other buffer, read after the last barrier)
    if constexpr (kOut) __syncthreads();

    bf16x8 vb[kCT];
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) vb[ct] = tr_operand<D + kTrPad>(&sm.v[0][0], 0, cw + 16 * ct, gi, l16);
    if constexpr (kOut) {
      // ---- O = diag(2^b) Q S + A V over this wavefront's columns
      f32x4 oacc[2][kCT];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) oacc[tt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        // B = S rows 32ks + {4gi..4gi+3, 16+4gi..16+4gi+3}; A = Q on the same rows
        bf16x8 bh[kCT], bl[kCT];
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          uint32_t h[4], l[4];
          split2(sacc[2 * ks][ct][0], sacc[2 * ks][ct][1], h[0], l[0]);
          split2(sacc[2 * ks][ct][2], sacc[2 * ks][ct][3], h[1], l[1]);
          split2(sacc[2 * ks + 1][ct][0], sacc[2 * ks + 1][ct][1], h[2], l[2]);
          split2(sacc[2 * ks + 1][ct][2], sacc[2 * ks + 1][ct][3], h[3], l[3]);
          bh[ct] = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
          bl[ct] = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const uint2 q0 = *reinterpret_cast<const uint2*>(&sm.u.r.q[16 * tt + l16][32 * ks + 4 * gi]);
          const uint2 q1 = *reinterpret_cast<const uint2*>(&sm.u.r.q[16 * tt + l16][32 * ks + 16 + 4 * gi]);
          const bf16x8 qa = __builtin_bit_cast(bf16x8, make_uint4(q0.x, q0.y, q1.x, q1.y));
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct) {
            oacc[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, bh[ct], oacc[tt][ct], 0, 0, 0);
            oacc[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, bl[ct], oacc[tt][ct], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gt = sm.g[buf][16 * tt + 4 * gi + e] * scale;
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct) oacc[tt][ct][e] *= gt;
        }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&sm.ah[16 * tt + l16][8 * gi]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&sm.al[16 * tt + l16][8 * gi]);
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          oacc[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, vb[ct], oacc[tt][ct], 0, 0, 0);
          oacc[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, vb[ct], oacc[tt][ct], 0, 0, 0);
        }
      }
      float* const ob = a.out + static_cast<int64_t>(pos) * row_elems + h * D + cw;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * tt + 4 * gi + e;
          if (t < n) {
#pragma unroll
            for (int ct = 0; ct < kCT; ++ct)
              __builtin_nontemporal_store(oacc[tt][ct][e], ob + t * row_elems + 16 * ct + l16);
          }
        }
    }

    // ---- S = 2^{b_{n-1}} S + K~^T V (in the scaled representation)
    gseg *= glast;
    if (lazy) {
      scale = cg;
    } else {
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) sacc[dt][ct] *= cg;
      scale = 1.0f;
    }
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const bf16x8 kh = tr_operand<D + kTrPad>(&sm.kh[0][0], 0, 16 * dt, gi, l16);
      const bf16x8 kl = tr_operand<D + kTrPad>(&sm.kl[0][0], 0, 16 * dt, gi, l16);
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        sacc[dt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, vb[ct], sacc[dt][ct], 0, 0, 0);
        sacc[dt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, vb[ct], sacc[dt][ct], 0, 0, 0);
      }
    }
    __syncthreads();                          // LDS is rewritten by the next chunk
  }

#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) sacc[dt][ct] *= scale;
  if constexpr (kMode == kSegState) {
    store_state(ws_state(seg));
    if (tid == 0) a.ws_gate[static_cast<int64_t>(seg) * H + h] = gseg;
  } else if (has_slot && j == nseg - 1) {
    store_state(slot_state);
  }
}

// ---- decode: the recurrent form, state streamed through registers ---------
//
// One workgroup per (request, head, 32-column slice of the state).  Thread
// (rg, cg) = (tid / 8, tid % 8) holds columns 4cg..4cg+3 of the slice in rows
// rg + 32 p; one row of the request at a time: S = gamma S + k^T v, then the
// thread's share of q S, summed over the 32 row groups in LDS.  Requests
// with several rows are handled row by row (correct, not fast).
constexpr int kDecSliceCols = 32;

template <int D>
__global__ __launch_bounds__(kThreads) void gated_retention_decode_kernel(RetArgs a) {
  constexpr int kSlices = D / kDecSliceCols;
  constexpr int kCG = kDecSliceCols / 4;      // float4 column groups of a slice
  constexpr int kRG = kThreads / kCG;         // row groups
  constexpr int kRows = D / kRG;              // rows per thread
  static_assert(kRows * kRG == D && kRows >= 1, "row split");
  __shared__ __attribute__((aligned(16))) float row_q[D];
  __shared__ __attribute__((aligned(16))) float row_k[D];
  __shared__ __attribute__((aligned(16))) float row_v[kDecSliceCols];
  __shared__ __attribute__((aligned(16))) float4 part[kRG][kCG];
  __shared__ float gate;

  const int tid = threadIdx.x;
  const int H = a.num_heads;
  const int slice = blockIdx.x % kSlices;
  const int rh = blockIdx.x / kSlices;
  const int r = rh / H;
  const int h = rh - r * H;
  int start, end;
  request_rows(a, r, start, end);
  if (end <= start) return;
  const int slot = a.slots[r];
  const bool has_slot = slot >= 0 && slot < a.num_slots;
  const int cg = tid % kCG;
  const int rg = tid / kCG;
  const int col0 = slice * kDecSliceCols;
  // float4 index of (row i, this thread's columns) within the head's state
  auto at = [&](int i) { return i * (D / 4) + col0 / 4 + cg; };
  float4* const st = has_slot ? reinterpret_cast<float4*>(a.state + (static_cast<int64_t>(slot) * H + h) * D * D)
                              : nullptr;
  float4 s[kRows];
#pragma unroll
  for (int p = 0; p < kRows; ++p)
    s[p] = has_slot ? yoco::load_stream_f4(reinterpret_cast<const float*>(st + at(rg + kRG * p)))
                    : make_float4(0.0f, 0.0f, 0.0f, 0.0f);

  for (int t = start; t < end; ++t) {
    const int64_t row = (static_cast<int64_t>(t) * H + h) * D;
    if (tid < D) {
      row_q[tid] = bf16_to_f32(a.q[row + tid]);
      row_k[tid] = bf16_to_f32(a.k[row + tid]);
    }
    if (tid < kDecSliceCols) row_v[tid] = bf16_to_f32(a.v[row + col0 + tid]);
    if (tid == 0) gate = a.gamma[static_cast<int64_t>(t) * H + h];
    __syncthreads();
    const float g = gate;
    const float4 vv = *reinterpret_cast<const float4*>(&row_v[4 * cg]);
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int p = 0; p < kRows; ++p) {
      const int i = rg + kRG * p;
      const float ki = row_k[i];
      const float qi = row_q[i];
      s[p].x = g * s[p].x + ki * vv.x;
      s[p].y = g * s[p].y + ki * vv.y;
      s[p].z = g * s[p].z + ki * vv.z;
      s[p].w = g * s[p].w + ki * vv.w;
      o.x += qi * s[p].x;
      o.y += qi * s[p].y;
      o.z += qi * s[p].z;
      o.w += qi * s[p].w;
    }
    part[rg][cg] = o;
    __syncthreads();
    if (tid < kDecSliceCols) {
      const float* pf = reinterpret_cast<const float*>(&part[0][0]);
      float sum = 0.0f;
#pragma unroll 8
      for (int g2 = 0; g2 < kRG; ++g2) sum += pf[g2 * kDecSliceCols + tid];
      a.out[row + col0 + tid] = sum;
    }
    __syncthreads();                          // rows and partials are rewritten for the next row
  }
  if (has_slot) {
#pragma unroll
    for (int p = 0; p < kRows; ++p) yoco::store_stream_f4(reinterpret_cast<float*>(st + at(rg + kRG * p)), s[p]);
  }
}

}  // namespace

namespace {

// The launch plan of a call: decode kernel, one run per request, or segments.
enum class RetPlan { kDecode, kWhole, kSegmented };

RetPlan plan_of(int32_t num_reqs, int32_t max_seqlen) {
  if (max_seqlen == 1) return RetPlan::kDecode;
  if ((max_seqlen > 0 && max_seqlen <= kSegRows) || num_reqs > kMaxSegReqs) return RetPlan::kWhole;
  return RetPlan::kSegmented;
}

// Segments a segmented launch may schedule: sum over requests of
// ceil(rows / kSegRows) <= num_reqs + num_tokens / kSegRows.
int64_t segment_bound(int32_t num_tokens, int32_t num_reqs) {
  return static_cast<int64_t>(num_reqs) + num_tokens / kSegRows;
}

}  // namespace

extern "C" int64_t yoco_gated_retention_workspace_size(int32_t num_tokens, int32_t num_reqs, int32_t num_heads,
                                                       int32_t head_dim, int32_t max_seqlen) {
  if (num_tokens < 0 || num_reqs < 0 || num_heads < 0 || head_dim <= 0) return -1;
  if (plan_of(num_reqs, max_seqlen) != RetPlan::kSegmented) return 0;
  const int64_t segs = segment_bound(num_tokens, num_reqs) * num_heads;
  const int64_t state_bytes = yoco::round_up(segs * head_dim * head_dim * 4, 256);
  return state_bytes + yoco::round_up(segs * 4, 256);
}

extern "C" int32_t yoco_gated_retention(int32_t dtype, const void* q, const void* k, const void* v,
                                        const float* gamma, int32_t num_tokens, int32_t num_heads,
                                        int32_t head_dim, const int32_t* cu_seqlens, int32_t num_reqs,
                                        int32_t max_seqlen, float* state, int32_t num_slots,
                                        const int32_t* state_indices, float* out, void* workspace,
                                        int64_t workspace_bytes, void* stream) {
  using namespace yoco;
  if (num_tokens < 0 || num_heads < 0 || num_reqs < 0 || num_slots < 0 || head_dim <= 0 || max_seqlen < 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gated_retention: negative count or non-positive head_dim");
  if (dtype != YOCO_DTYPE_BF16 && dtype != YOCO_DTYPE_F32)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gated_retention: dtype %d is not bf16 or fp32", dtype);
  if (dtype != YOCO_DTYPE_BF16)
    return fail(YOCO_ERR_UNSUPPORTED, "gated_retention: only bf16 q/k/v have a kernel");
  if (head_dim != 64 && head_dim != 128)
    return fail(YOCO_ERR_UNSUPPORTED, "gated_retention: head_dim %d (64 or 128 supported)", head_dim);
  if (num_reqs == 0 || num_heads == 0) return YOCO_OK;
  if (cu_seqlens == nullptr || state_indices == nullptr || (num_slots > 0 && state == nullptr) ||
      (num_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || gamma == nullptr || out == nullptr)))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gated_retention: null pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gated_retention: q, k, v and state must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0 || (reinterpret_cast<uintptr_t>(gamma) & 3u) != 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gated_retention: out and gamma must be 4-byte aligned");
  const RetPlan plan = plan_of(num_reqs, max_seqlen);
  const int64_t items = plan == RetPlan::kSegmented ? segment_bound(num_tokens, num_reqs)
                       : plan == RetPlan::kDecode  ? static_cast<int64_t>(num_reqs) * (head_dim / kDecSliceCols)
                                                   : num_reqs;
  if (static_cast<int64_t>(num_heads) * head_dim >= (int64_t(1) << 26))
    return fail(YOCO_ERR_UNSUPPORTED, "gated_retention: num_heads * head_dim must stay below 2^26");
  const int64_t blocks = items * num_heads;
  if (blocks > 0x7fffffff) return fail(YOCO_ERR_UNSUPPORTED, "gated_retention: too many (request, head) pairs");
  const int64_t need = yoco_gated_retention_workspace_size(num_tokens, num_reqs, num_heads, head_dim, max_seqlen);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return fail(YOCO_ERR_WORKSPACE_TOO_SMALL, "gated_retention: workspace of %lld bytes needed (16-byte aligned)",
                static_cast<long long>(need));
  if (num_tokens == 0) return YOCO_OK;
  if (yoco_validation_enabled()) {
    std::vector<int32_t> cu, idx;
    bool skip = false;
    int32_t st = fetch_indices(cu_seqlens, int64_t{num_reqs} + 1, static_cast<hipStream_t>(stream), cu, skip,
                               "gated_retention");
    if (st == YOCO_OK)
      st = fetch_indices(state_indices, num_reqs, static_cast<hipStream_t>(stream), idx, skip, "gated_retention");
    if (st != YOCO_OK) return st;
    if (!skip && (yoco_validate_offsets(cu.data(), num_reqs, num_tokens) != YOCO_OK ||
                  yoco_validate_state_indices(idx.data(), num_reqs, num_slots) != YOCO_OK))
      return YOCO_ERR_INVALID_ARGUMENT;
  }

  RetArgs args;
  args.q = static_cast<const uint16_t*>(q);
  args.k = static_cast<const uint16_t*>(k);
  args.v = static_cast<const uint16_t*>(v);
  args.gamma = gamma;
  args.cu = cu_seqlens;
  args.slots = state_indices;
  args.state = state;
  args.out = out;
  args.ws_state = nullptr;
  args.ws_gate = nullptr;
  if (need > 0) {
    const int64_t segs = segment_bound(num_tokens, num_reqs) * num_heads;
    args.ws_state = static_cast<float*>(workspace);
    args.ws_gate = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            round_up(segs * head_dim * head_dim * 4, 256));
  }
  args.num_tokens = num_tokens;
  args.num_heads = num_heads;
  args.num_slots = num_slots;
  args.num_reqs = num_reqs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  clear_launch_error();
  auto launch = [&](auto d_tag) {
    constexpr int D = decltype(d_tag)::value;
    switch (plan) {
      case RetPlan::kDecode:
        hipLaunchKernelGGL(gated_retention_decode_kernel<D>, grid, block, 0, s, args);
        break;
      case RetPlan::kWhole:
        hipLaunchKernelGGL((gated_retention_kernel<D, kWhole>), grid, block, 0, s, args);
        break;
      case RetPlan::kSegmented:
        hipLaunchKernelGGL((gated_retention_kernel<D, kSegState>), grid, block, 0, s, args);
        hipLaunchKernelGGL((gated_retention_kernel<D, kSegFull>), grid, block, 0, s, args);
        break;
    }
  };
  if (head_dim == 64)
    launch(std::integral_constant<int, 64>());
  else
    launch(std::integral_constant<int, 128>());
  return launch_result("gated_retention");
}
