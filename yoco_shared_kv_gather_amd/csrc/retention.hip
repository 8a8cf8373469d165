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
// which is the recurrence unrolled over the chunk.  A decode step is the
// same with n = 1, so one kernel serves prefill and decode.
//
// One workgroup per (request, head) walks that request's tokens chunk by
// chunk with the head's fp32 state resident in registers (wavefront w owns
// value columns [w D/4, (w+1) D/4) for all key rows, in the MFMA accumulator
// layout), so the state is read from and written to HBM once per call.  Per
// chunk:
//   stage    Q, K, V rows (bf16) in LDS row-major; K~^T = (w_s k_s)^T split
//            into bf16 high and low parts and V^T transposed from there; the
//            per-token decay terms from one wavefront's prefix sum;
//   A = QK^T three 16x16 causal tiles (v_mfma_f32_16x16x32_bf16), each
//            scaled by 2^{b_t - b_s}, stored as bf16 high + low parts;
//   O        Q S (the state split into bf16 high + low in registers), rows
//            scaled by 2^{b_t}, plus A V;
//   S        2^{b_{n-1}} S + K~^T V.
// The next chunk's rows are loaded into registers while the current one is
// computed.  q, k and v are exact bf16 operands; every fp32 operand (state,
// A, K~) enters as two bf16 parts (~17 significant bits); sums are fp32.
// log2 gamma is clamped at -64, so a zero gate weighs 2^-64 instead of 0.

#include "yoco_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kC = 32;                  // tokens per chunk
constexpr int kRowPad = 8;              // bf16 elements of padding per LDS row
constexpr float kMinLog2Gate = -64.0f;

struct RetArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* gamma;
  const int32_t* cu;
  const int32_t* slots;
  float* state;
  float* out;
  int32_t num_tokens;
  int32_t num_heads;
  int32_t num_slots;
};

template <int D>
struct __attribute__((aligned(16))) RetSmem {
  uint16_t q[kC][D + kRowPad];          // row-major chunk rows
  uint16_t k[kC][D + kRowPad];
  uint16_t v[kC][D + kRowPad];
  uint16_t kth[D][kC + kRowPad];        // (w_s k_s)^T, bf16 high part
  uint16_t ktl[D][kC + kRowPad];        // low part
  uint16_t vt[D][kC + kRowPad];         // V^T
  uint16_t ah[kC][kC + kRowPad];        // decayed causal Q K^T, high part
  uint16_t al[kC][kC + kRowPad];        // low part
  float b[kC];                          // inclusive prefix of log2 gamma
  float g[kC];                          // 2^{b_t}
  float w[kC];                          // 2^{b_{n-1} - b_s}
};

__device__ __forceinline__ uint16_t bf16_bits(__bf16 h) { return __builtin_bit_cast(uint16_t, h); }

// x = hi + lo with hi, lo bf16 (hi the nearest bf16 to x).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gated_retention_kernel(RetArgs a) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int kCW = D / kWaves;             // value columns per wavefront
  constexpr int kCT = kCW / 16;               // 16-column tiles per wavefront
  constexpr int kDT = D / 16;                 // 16-row tiles of the state (key rows)
  constexpr int kKS = D / 32;                 // MFMA k-steps over head_dim
  constexpr int kRowChunks = D / 8;           // 16-byte chunks per row
  constexpr int kLoads = kC * kRowChunks / kThreads;   // row chunks per thread per matrix
  constexpr int kTasks = D * (kC / 8) / kThreads;      // transpose tasks per thread
  static_assert(kLoads >= 1 && kC * kRowChunks % kThreads == 0, "row staging split");
  static_assert(kTasks >= 1 && D * (kC / 8) % kThreads == 0, "transpose split");
  using Smem = RetSmem<D>;
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int gi = lane >> 4;
  const int H = a.num_heads;
  const int r = blockIdx.x / H;
  const int h = blockIdx.x - r * H;

  const int start = min(max(a.cu[r], 0), a.num_tokens);
  const int end = min(max(a.cu[r + 1], start), a.num_tokens);
  if (end <= start) return;                   // no rows: the state is left as it is
  const int slot = a.slots[r];
  const bool has_slot = slot >= 0 && slot < a.num_slots;
  const int cw = wave * kCW;

  // ---- the state: S[16dt + 4gi + e][cw + 16ct + l16] in sacc[dt][ct][e]
  f32x4 sacc[kDT][kCT];
  float* const st = has_slot ? a.state + (static_cast<int64_t>(slot) * H + h) * D * D : nullptr;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sacc[dt][ct][e] = has_slot ? st[(16 * dt + 4 * gi + e) * D + cw + 16 * ct + l16] : 0.0f;

  // the strictly upper tile of A is never written by the chunk loop
  for (int i = tid; i < 16 * 16; i += kThreads) {
    sm.ah[i >> 4][16 + (i & 15)] = 0;
    sm.al[i >> 4][16 + (i & 15)] = 0;
  }

  // ---- chunk rows in registers: thread chunk c = tid + 256 i covers row
  // c / kRowChunks, elements 8 (c % kRowChunks) .. +7
  uint4 rq[kLoads], rk[kLoads], rv[kLoads];
  float rg = 1.0f;                            // wavefront 0, lanes < 32: the token's gate
  auto load_chunk = [&](int pos) {
    const int n = min(kC, end - pos);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i;
      const int s = c / kRowChunks;
      const int cc = c - s * kRowChunks;
      if (s < n) {
        const int64_t off = ((static_cast<int64_t>(pos + s) * H + h) * D + 8 * cc);
        rq[i] = *reinterpret_cast<const uint4*>(a.q + off);
        rk[i] = *reinterpret_cast<const uint4*>(a.k + off);
        rv[i] = *reinterpret_cast<const uint4*>(a.v + off);
      } else {
        rq[i] = rk[i] = rv[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (wave == 0) rg = lane < n ? a.gamma[static_cast<int64_t>(pos + lane) * H + h] : 1.0f;
  };

  load_chunk(start);
  for (int pos = start; pos < end; pos += kC) {
    const int n = min(kC, end - pos);
    // ---- stage the rows; decay terms from wavefront 0
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i;
      const int s = c / kRowChunks;
      const int cc = c - s * kRowChunks;
      *reinterpret_cast<uint4*>(&sm.q[s][8 * cc]) = rq[i];
      *reinterpret_cast<uint4*>(&sm.k[s][8 * cc]) = rk[i];
      *reinterpret_cast<uint4*>(&sm.v[s][8 * cc]) = rv[i];
    }
    if (wave == 0) {
      float lg = lane < n ? fmaxf(__builtin_amdgcn_logf(rg), kMinLog2Gate) : 0.0f;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const float t = __shfl_up(lg, off, 64);
        if ((lane & 31) >= off) lg += t;
      }
      const float blast = __shfl(lg, n - 1, 64);
      if (lane < kC) {
        sm.b[lane] = lg;
        sm.g[lane] = __builtin_amdgcn_exp2f(lg);
        sm.w[lane] = lane < n ? __builtin_amdgcn_exp2f(blast - lg) : 0.0f;
      }
    }
    // the next chunk's rows travel while this one is computed
    if (pos + kC < end) load_chunk(pos + kC);
    __syncthreads();

    // ---- transposed operands: K~^T (high, low) and V^T; task c = tid + 256 i
    // is key/value row c % D, tokens 8 (c / D) .. +7
#pragma unroll
    for (int i = 0; i < kTasks; ++i) {
      const int c = tid + kThreads * i;
      const int d = c % D;
      const int s0 = 8 * (c / D);
      bf16x8 hi, lo;
      uint32_t vw[4];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = sm.w[s0 + j] * bf16_to_f32(sm.k[s0 + j][d]);
        __bf16 xh, xl;
        split_bf16(x, xh, xl);
        hi[j] = xh;
        lo[j] = xl;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vw[j] = static_cast<uint32_t>(sm.v[s0 + 2 * j][d]) | (static_cast<uint32_t>(sm.v[s0 + 2 * j + 1][d]) << 16);
      *reinterpret_cast<bf16x8*>(&sm.kth[d][s0]) = hi;
      *reinterpret_cast<bf16x8*>(&sm.ktl[d][s0]) = lo;
      *reinterpret_cast<uint4*>(&sm.vt[d][s0]) = make_uint4(vw[0], vw[1], vw[2], vw[3]);
    }
    // ---- A = Q K^T, causal tiles (t-tile, s-tile) = (0,0), (1,0), (1,1)
    if (wave < 3) {
      const int tt = (wave + 1) >> 1;
      const int ts = wave >> 1;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&sm.q[16 * tt + l16][32 * ks + 8 * gi]);
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&sm.k[16 * ts + l16][32 * ks + 8 * gi]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kb, acc, 0, 0, 0);
      }
      const int s = 16 * ts + l16;
      const float bs = sm.b[s];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tt + 4 * gi + e;
        const float val = (s <= t && t < n) ? acc[e] * __builtin_amdgcn_exp2f(sm.b[t] - bs) : 0.0f;
        __bf16 vh, vl;
        split_bf16(val, vh, vl);
        sm.ah[t][s] = bf16_bits(vh);
        sm.al[t][s] = bf16_bits(vl);
      }
    }
    __syncthreads();

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
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          __bf16 h0, l0, h1, l1;
          split_bf16(sacc[2 * ks][ct][e], h0, l0);
          split_bf16(sacc[2 * ks + 1][ct][e], h1, l1);
          bh[ct][e] = h0;
          bl[ct][e] = l0;
          bh[ct][4 + e] = h1;
          bl[ct][4 + e] = l1;
        }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const uint2 q0 = *reinterpret_cast<const uint2*>(&sm.q[16 * tt + l16][32 * ks + 4 * gi]);
        const uint2 q1 = *reinterpret_cast<const uint2*>(&sm.q[16 * tt + l16][32 * ks + 16 + 4 * gi]);
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
        const float gt = sm.g[16 * tt + 4 * gi + e];
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) oacc[tt][ct][e] *= gt;
      }
    bf16x8 vb[kCT];
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) vb[ct] = *reinterpret_cast<const bf16x8*>(&sm.vt[cw + 16 * ct + l16][8 * gi]);
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
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tt + 4 * gi + e;
        if (t < n) {
          float* o = a.out + (static_cast<int64_t>(pos + t) * H + h) * D + cw + l16;
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct) o[16 * ct] = oacc[tt][ct][e];
        }
      }

    // ---- S = 2^{b_{n-1}} S + K~^T V
    const float glast = sm.g[n - 1];
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const bf16x8 kh = *reinterpret_cast<const bf16x8*>(&sm.kth[16 * dt + l16][8 * gi]);
      const bf16x8 kl = *reinterpret_cast<const bf16x8*>(&sm.ktl[16 * dt + l16][8 * gi]);
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        sacc[dt][ct] *= glast;
        sacc[dt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, vb[ct], sacc[dt][ct], 0, 0, 0);
        sacc[dt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, vb[ct], sacc[dt][ct], 0, 0, 0);
      }
    }
    __syncthreads();                          // LDS is rewritten by the next chunk
  }

  if (has_slot) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[(16 * dt + 4 * gi + e) * D + cw + 16 * ct + l16] = sacc[dt][ct][e];
  }
}

}  // namespace

extern "C" int32_t yoco_gated_retention(int32_t dtype, const void* q, const void* k, const void* v,
                                        const float* gamma, int32_t num_tokens, int32_t num_heads,
                                        int32_t head_dim, const int32_t* cu_seqlens, int32_t num_reqs,
                                        float* state, int32_t num_slots, const int32_t* state_indices,
                                        float* out, void* stream) {
  using namespace yoco;
  if (num_tokens < 0 || num_heads < 0 || num_reqs < 0 || num_slots < 0 || head_dim <= 0)
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
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gated_retention: q, k and v must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(state) & 3u) != 0 || (reinterpret_cast<uintptr_t>(out) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(gamma) & 3u) != 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "gated_retention: state, out and gamma must be 4-byte aligned");
  const int64_t blocks = static_cast<int64_t>(num_reqs) * num_heads;
  if (blocks > 0x7fffffff) return fail(YOCO_ERR_UNSUPPORTED, "gated_retention: too many (request, head) pairs");
  if (num_tokens == 0) return YOCO_OK;

  RetArgs args;
  args.q = static_cast<const uint16_t*>(q);
  args.k = static_cast<const uint16_t*>(k);
  args.v = static_cast<const uint16_t*>(v);
  args.gamma = gamma;
  args.cu = cu_seqlens;
  args.slots = state_indices;
  args.state = state;
  args.out = out;
  args.num_tokens = num_tokens;
  args.num_heads = num_heads;
  args.num_slots = num_slots;
  hipStream_t s = static_cast<hipStream_t>(stream);
  clear_launch_error();
  if (head_dim == 64)
    hipLaunchKernelGGL(gated_retention_kernel<64>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, args);
  else
    hipLaunchKernelGGL(gated_retention_kernel<128>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, args);
  return launch_result("gated_retention");
}
