// yoco_kv_append: RMSNorm + the shared K/V projection, written once per token
// into the paged cache.
//
// "YOCO_论文与推理数据流详解" §3 (architecture flowchart) and §10.3: from the
// self-decoder output M the model computes K^ = LN(M) W_K and V^ = LN(M) W_V
// once per token and appends that pair to the single global cache; no cross
// layer appends anything.  LN is taken as RMSNorm,
//     xhat = x * rsqrt(mean(x^2) + eps) * w_rms,
// and the row scale rsqrt(...) commutes with the projection:
//     K^_t = rsqrt(mean(x_t^2) + eps) * (W_K diag(w_rms)) x_t.
//
// bf16 path (matrix cores), two shapes:
//   * many tokens (prefill): fold W' = bf16(W diag(w_rms)) for [W_K; W_V]
//     once into the workspace, then one MFMA GEMM C[T][2*Hkv*D] = x W'^T
//     with v_mfma_f32_16x16x32_bf16 (fp32 accumulation) in 128x256 tiles;
//     the same pass sums x^2 per row from the staged A tiles, and the
//     epilogue multiplies by the row's rsqrt, rounds to bf16 (nearest even)
//     and scatters each [Hkv][D] row to its slot.
//   * few tokens (decode, T <= 64): reading the weights is the whole cost,
//     so every workgroup takes 16 output features for all tokens and its
//     eight wavefronts split the hidden dimension; the RMS weight multiplies the
//     few activation rows instead (one bf16 rounding of x*w, as the fold
//     rounds W*w once), and no fold pass or workspace is used.
// fp32 path: one workgroup per token, fp32 throughout.
//
// 8-bit cache ("KV cache memory systems", section "Quantized cache changes
// attention inputs"; "YOCO_论文与推理数据流详解" §18.2: quantize the shared
// K/V once and let every cross layer reuse it): FP8 E4M3 codes with one fp32
// scale per (token, KV head), s = max|x| / 448, code = E4M3(x / s) rounded to
// nearest even, both divisions in fp32 on the fp32 projection.  The tiled
// GEMM quantizes in its epilogue; the few-token and fp32 kernels write each
// token's fp32 K^/V^ row to a workspace, and a quantizing scatter stores the
// codes.  That scatter is also the public yoco_kv_scatter (rows computed
// elsewhere).

#include <cmath>

#include "yoco_internal.h"

namespace {

using yoco::bf16_hi;
using yoco::bf16_lo;
using yoco::f32_to_bf16_rne;

// Largest of x over the 16 lanes of each DPP row (lanes 16r..16r+15): swap
// neighbours, then pairs, then mirror within each half row and within the
// row; every lane ends with the row's value.
__device__ __forceinline__ uint32_t row16_max(uint32_t x) {
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0xB1, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x4E, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x141, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x140, 0xF, 0xF, false)));
  return x;
}

// ---- fold W' = W diag(w_rms) -------------------------------------------------

__global__ __launch_bounds__(256) void fold_rms_weight_kernel(const uint4* __restrict__ w_k,
                                                              const uint4* __restrict__ w_v,
                                                              const uint4* __restrict__ w_rms,
                                                              uint4* __restrict__ w_out, int64_t half_chunks,
                                                              int hidden_chunks) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= 2 * half_chunks) return;
  const uint4 src = c < half_chunks ? w_k[c] : w_v[c - half_chunks];
  const uint4 sc = w_rms[c % hidden_chunks];
  const uint32_t* s = reinterpret_cast<const uint32_t*>(&src);
  const uint32_t* m = reinterpret_cast<const uint32_t*>(&sc);
  uint4 res;
  uint32_t* o = reinterpret_cast<uint32_t*>(&res);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = f32_to_bf16_rne(bf16_lo(s[i]) * bf16_lo(m[i]));
    const uint32_t hi = f32_to_bf16_rne(bf16_hi(s[i]) * bf16_hi(m[i]));
    o[i] = lo | (hi << 16);
  }
  w_out[c] = res;
}

// ---- bf16 MFMA GEMM with RMS row scale and slot scatter ------------------------

constexpr int kBM = 128;                     // tokens per workgroup tile
constexpr int kBN = 256;                     // output features per workgroup tile
constexpr int kBK = 32;
constexpr int kLdsStride = kBK;              // bf16 elements per staged row (4 chunks of 16 bytes, swizzled)
static_assert(kBK == 32, "the row swizzle covers four 16-byte chunks");
constexpr int kStage = (kBM + kBN) * kLdsStride;
constexpr int kOutStride = kBN + 8;          // bf16 elements per row of the staged output tile
constexpr int kGemmThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct AppendArgs {
  const uint16_t* x;          // [T][H]
  const uint16_t* w;          // folded [2*Hkv*D][H]
  const int32_t* slots;       // [T]
  uint16_t* k_cache;
  uint16_t* v_cache;
  int32_t num_tokens;
  int32_t hidden;
  int32_t out_half;           // Hkv * D
  int32_t head_dim;
  int32_t block_size;
  int32_t bs_shift;
  int32_t num_kv_heads;
  int32_t n_tiles;            // ceil(2 * out_half / kBN)
  int32_t num_tiles;          // token tiles x feature tiles
  int32_t tiles_per_xcd;      // ceil(num_tiles / 8)
  int64_t num_slots;          // num_blocks * block_size
  float inv_hidden;
  float eps;
  float* k_scale;             // FP8 cache: [num_blocks][Hkv][bs] scales (caches hold bytes), else nullptr
  float* v_scale;
};

// Staged rows hold their four 16-byte chunks in the order chunk ^ swz(row):
// a fragment read (16 consecutive rows, one chunk) then touches distinct bank
// groups in every 8 or 16 consecutive lanes (a padded row of 80 bytes left a
// third of the LDS cycles in bank conflicts on gfx950).
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// One workgroup: 128 tokens x 256 output features, four wavefronts of 64 x 128
// (4 x 8 MFMA tiles of 16x16), K step 32, two workgroups per compute unit
// (K step 64 left one, with nothing to cover its LDS waits).  Workgroup b runs
// on XCD b % 8, and XCD x takes the tiles [x*per, (x+1)*per) of the order
// (token tile, feature tile) with the feature tile fastest: the feature
// tiles of one activation panel run on one XCD at about the same time and
// share the panel through its L2 (with the feature tile = b % 8, every panel
// went to all eight XCDs, 3.5 GB of L2 misses for 0.4 GB of activations on
// the mixed step).  Global -> registers -> LDS staging, two LDS stages, one barrier per
// K step.  The epilogue scales by the row's rsqrt, rounds to bf16 into LDS and
// writes each token's features as 16-byte chunks to its slot.  With kQD > 0
// (the head_dim of an FP8 cache) the epilogue quantizes instead: a tile holds
// whole heads (256 is a multiple of every head_dim), and for head_dim 128 a
// 16-lane DPP row of a wavefront holds every column of its rows' head, so
// the head's largest magnitude is a max over the lane's 8 values and a DPP
// row (two heads per wavefront for 64; for 256 the two column halves meet in
// LDS).  s = max / 448 and code = E4M3(y / s) in fp32 on the scaled fp32
// projection y, exactly as the quantizing scatter would (the quotient's code
// mostly without the division, as e4m3_of_quotient explains); codes go through an
// LDS byte tile to 16-byte stores, scales straight from the lanes.
template <int kQD>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2))) void kv_append_mfma_kernel(AppendArgs a) {
  constexpr int kLdsElems = 2 * kStage > kBM * kOutStride ? 2 * kStage : kBM * kOutStride;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems];
  __shared__ float row_scale[kBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;            // 64-row half of the tile
  const int wn = wave & 1;             // 128-column half of the tile
  const int tile = static_cast<int>(blockIdx.x % 8) * a.tiles_per_xcd + static_cast<int>(blockIdx.x / 8);
  if (tile >= a.num_tiles) return;
  const int m0 = (tile / a.n_tiles) * kBM;
  const int n0 = (tile % a.n_tiles) * kBN;
  const int n_total = 2 * a.out_half;

  // Staging map: thread moves chunk kc (8 bf16) of A rows rbase+kRp*i
  // (i<kAP) and of B rows rbase+kRp*i (i<kBP).
  constexpr int kCk = kBK / 8;                 // 16-byte chunks per staged row
  constexpr int kRp = kGemmThreads / kCk;      // rows per staging pass
  constexpr int kAP = kBM / kRp, kBP = kBN / kRp;
  const int kc = tid % kCk;
  const int rbase = tid / kCk;
  // Two tiles in flight, in two register sets.  Rows past the last token and
  // features past the last one load the last valid row instead: their
  // products land in outputs that are never stored, so the loads need no
  // branch or select (either would make the compiler wait for them at once).
  struct TileRegs {
    uint4 a[kAP], b[kBP];
  };
  TileRegs r0, r1;
  const uint16_t* arow[kAP];
  const uint16_t* brow[kBP];
#pragma unroll
  for (int i = 0; i < kAP; ++i)
    arow[i] = a.x + static_cast<int64_t>(min(m0 + rbase + kRp * i, a.num_tokens - 1)) * a.hidden + kc * 8;
#pragma unroll
  for (int i = 0; i < kBP; ++i)
    brow[i] = a.w + static_cast<int64_t>(min(n0 + rbase + kRp * i, n_total - 1)) * a.hidden + kc * 8;
  float sumsq[kAP];
#pragma unroll
  for (int i = 0; i < kAP; ++i) sumsq[i] = 0.0f;

  auto load_tile = [&](TileRegs& r, int k0) {
#pragma unroll
    for (int i = 0; i < kAP; ++i) r.a[i] = *reinterpret_cast<const uint4*>(arow[i] + k0);
#pragma unroll
    for (int i = 0; i < kBP; ++i) r.b[i] = *reinterpret_cast<const uint4*>(brow[i] + k0);
  };
  auto store_tile = [&](const TileRegs& r, int stage, bool real) {
    uint16_t* as = lds + stage * kStage;
    uint16_t* bs = as + kBM * kLdsStride;
#pragma unroll
    for (int i = 0; i < kAP; ++i) {
      const int row = rbase + kRp * i;
      *reinterpret_cast<uint4*>(&as[row * kLdsStride + ((kc ^ swz(row)) * 8)]) = r.a[i];
      // a repeated tile adds nothing (one select per chunk, not a branch:
      // the stores, loads and products of a half-iteration stay one block
      // the scheduler can interleave; a select per element cost 0.8% on
      // mixed48's 67,387 rows, 884.5 -> 877.7 us)
      const uint32_t* u = reinterpret_cast<const uint32_t*>(&r.a[i]);
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(u[e]);
        const float hi = bf16_hi(u[e]);
        part = fmaf(lo, lo, part);
        part = fmaf(hi, hi, part);
      }
      sumsq[i] += real ? part : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kBP; ++i) {
      const int row = rbase + kRp * i;
      *reinterpret_cast<uint4*>(&bs[row * kLdsStride + ((kc ^ swz(row)) * 8)]) = r.b[i];
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int ktiles = a.hidden / kBK;
  const int frag_row = lane & 15;
  // chunk lane/16 of rows congruent to frag_row mod 16 (t*16 and the
  // wavefront's offset leave the swizzle bits alone)
  const int frag_k = ((lane >> 4) ^ swz(frag_row)) * 8;
  auto mma = [&](int stage) {
    const uint16_t* as = lds + stage * kStage;
    const uint16_t* bs = as + kBM * kLdsStride;
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 32) {
      bf16x8 af[4], bf[8];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        af[t] = *reinterpret_cast<const bf16x8*>(&as[(wm * 64 + t * 16 + frag_row) * kLdsStride + ks + frag_k]);
#pragma unroll
      for (int t = 0; t < 8; ++t)
        bf[t] = *reinterpret_cast<const bf16x8*>(&bs[(wn * 128 + t * 16 + frag_row) * kLdsStride + ks + frag_k]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // Tile kt is in LDS stage kt&1 while tiles kt+1 and kt+2 are in flight in
  // the register sets (tile j in set j&1).  Past the last K tile the loads
  // repeat the last one: every iteration issues the same loads in the same
  // order, so the wait before a set is staged covers that set only, not the
  // one loaded after it.
  auto kofs = [&](int kt) { return min(kt, ktiles - 1) * kBK; };
  load_tile(r0, 0);
  load_tile(r1, kofs(1));
  store_tile(r0, 0, true);
  load_tile(r0, kofs(2));
  __syncthreads();
  // hidden is a multiple of 64, so ktiles is even and both halves of every
  // iteration stage a real tile, except the last half, which stages a repeat
  // of the last tile into stage 0 (never read, its squares not added).  A
  // half is one branch-free block, ordered: the fragment reads, then the 32
  // products with the next tile's LDS stores and global loads spread
  // between them (81k tokens: 1050 -> 950 us; spreading the fragment reads
  // too, which keeps the stores behind the last read, 1014 us).
  static_assert(4 * (kAP + kBP) <= 32, "one store and one load per four products");
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);   // fragment reads
#pragma unroll
    for (int g = 0; g < kAP + kBP; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // products
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // one LDS store
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 32 - 4 * (kAP + kBP), 0);
  };
  for (int kt = 0; kt < ktiles; kt += 2) {
    mma(0);
    store_tile(r1, 1, true);
    load_tile(r1, kofs(kt + 3));
    interleave();
    __syncthreads();
    mma(1);
    store_tile(r0, 0, kt + 2 < ktiles);
    load_tile(r0, kofs(kt + 4));
    interleave();
    __syncthreads();
  }

  // Row scale rsqrt(mean(x^2) + eps): add the kCk partial sums of each row.
#pragma unroll
  for (int i = 0; i < kAP; ++i) {
    float v = sumsq[i];
#pragma unroll
    for (int off = 1; off < kCk; off <<= 1) v += __shfl_xor(v, off, 64);
    if (kc == 0) row_scale[rbase + kRp * i] = 1.0f / sqrtf(v * a.inv_hidden + a.eps);
  }
  __syncthreads();

  if constexpr (kQD > 0) {
    constexpr int kHeadsPerWave = kQD >= 128 ? 1 : 128 / kQD;   // heads in a wavefront's 128 columns
    constexpr int kJPerHead = kQD >= 128 ? 8 : kQD / 16;        // 16-column MFMA tiles per head in a wavefront
    constexpr int kCodeStride = kBN + 16;                      // bytes per row of the code tile
    uint8_t* ct = reinterpret_cast<uint8_t*>(lds);
    float* hmax = reinterpret_cast<float*>(ct + kBM * kCodeStride);   // [2][kBM], head_dim 256 only
    static_assert(kBM * kCodeStride + 2 * kBM * sizeof(float) <= sizeof(lds), "code tile exceeds the staging LDS");
    uint32_t mb[4][4][kHeadsPerWave];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int lrow = wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        const float sc = row_scale[lrow];
#pragma unroll
        for (int hw = 0; hw < kHeadsPerWave; ++hw) {
          uint32_t m = 0;
#pragma unroll
          for (int jj = 0; jj < kJPerHead; ++jj) {
            const int j = hw * kJPerHead + jj;
            acc[i][j][e] *= sc;
            m = max(m, __float_as_uint(acc[i][j][e]) & 0x7fffffffu);
          }
          mb[i][e][hw] = row16_max(m);
        }
      }
    if constexpr (kQD == 256) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((lane & 15) == 0) hmax[wn * kBM + wm * 64 + i * 16 + (lane >> 4) * 4 + e] = __uint_as_float(mb[i][e][0]);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int lrow = wm * 64 + i * 16 + (lane >> 4) * 4 + e;
          mb[i][e][0] = max(__float_as_uint(hmax[lrow]), __float_as_uint(hmax[kBM + lrow]));
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int lrow = wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        const int t = m0 + lrow;
#pragma unroll
        for (int hw = 0; hw < kHeadsPerWave; ++hw) {
          const float s = __uint_as_float(mb[i][e][hw]) / 448.0f;
          const bool finite = mb[i][e][hw] < 0x7f800000u;
          const float r = finite && s > 0.0f ? 1.0f / s : 0.0f;
#pragma unroll
          for (int jj = 0; jj < kJPerHead; ++jj) {
            const int j = hw * kJPerHead + jj;
            const uint32_t code = !finite ? 0x7fu : (s == 0.0f ? 0u : yoco::e4m3_of_quotient(acc[i][j][e], s, r));
            ct[lrow * kCodeStride + wn * 128 + j * 16 + (lane & 15)] = static_cast<uint8_t>(code);
          }
          const int col0 = n0 + wn * 128 + hw * kQD;
          if ((lane & 15) == 0 && (kQD < 256 || wn == 0) && t < a.num_tokens && col0 < n_total) {
            const int64_t slot = a.slots[t];
            if (slot >= 0 && slot < a.num_slots) {
              const bool is_v = col0 >= a.out_half;
              const int h = (is_v ? col0 - a.out_half : col0) / kQD;
              const int64_t row = ((slot >> a.bs_shift) * a.num_kv_heads + h) * a.block_size + (slot & (a.block_size - 1));
              (is_v ? a.v_scale : a.k_scale)[row] = s;
            }
          }
        }
      }
    __syncthreads();
    // Each token's codes, 16 bytes (16 features, inside one head) at a time.
    for (int c = tid; c < kBM * (kBN / 16); c += kGemmThreads) {
      const int lrow = c / (kBN / 16);
      const int lcol = (c % (kBN / 16)) * 16;
      const int t = m0 + lrow;
      const int col = n0 + lcol;
      if (t >= a.num_tokens || col >= n_total) continue;
      const int64_t slot = a.slots[t];
      if (slot < 0 || slot >= a.num_slots) continue;
      const bool is_v = col >= a.out_half;
      const int hd = is_v ? col - a.out_half : col;
      const int h = hd / kQD;
      const int d = hd - h * kQD;
      uint8_t* cache = reinterpret_cast<uint8_t*>(is_v ? a.v_cache : a.k_cache);
      const int64_t dst = (((slot >> a.bs_shift) * a.num_kv_heads + h) * a.block_size + (slot & (a.block_size - 1))) *
                              kQD + d;
      *reinterpret_cast<uint4*>(cache + dst) = *reinterpret_cast<const uint4*>(&ct[lrow * kCodeStride + lcol]);
    }
    return;
  }

  // Scaled, rounded tile into LDS (the staging buffers are free now).  Lane
  // holds rows 4*(lane/16)+0..3 of column lane%16 of each 16x16 tile.
  uint16_t* ot = lds;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int lrow = wm * 64 + i * 16 + (lane >> 4) * 4 + e;
      const float sc = row_scale[lrow];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int lcol = wn * 128 + j * 16 + (lane & 15);
        ot[lrow * kOutStride + lcol] = static_cast<uint16_t>(yoco::pack_bf16x2(acc[i][j][e] * sc, 0.0f));
      }
    }
  __syncthreads();

  // Each token's features, 16 bytes (8 features, inside one head) at a time.
  for (int c = tid; c < kBM * (kBN / 8); c += kGemmThreads) {
    const int lrow = c / (kBN / 8);
    const int lcol = (c % (kBN / 8)) * 8;
    const int t = m0 + lrow;
    const int col = n0 + lcol;
    if (t >= a.num_tokens || col >= n_total) continue;
    const int64_t slot = a.slots[t];
    if (slot < 0 || slot >= a.num_slots) continue;
    const bool is_v = col >= a.out_half;
    const int hd = is_v ? col - a.out_half : col;
    const int h = hd / a.head_dim;
    const int d = hd - h * a.head_dim;
    uint16_t* cache = is_v ? a.v_cache : a.k_cache;
    const int64_t dst = (((slot >> a.bs_shift) * a.num_kv_heads + h) * a.block_size + (slot & (a.block_size - 1))) *
                            a.head_dim + d;
    *reinterpret_cast<uint4*>(cache + dst) = *reinterpret_cast<const uint4*>(&ot[lrow * kOutStride + lcol]);
  }
}

// ---- fp32 path -----------------------------------------------------------------

constexpr int kF32Threads = 256;

__global__ __launch_bounds__(kF32Threads) void kv_append_f32_kernel(
    const float* __restrict__ x, int hidden, const float* __restrict__ w_rms, float eps,
    const float* __restrict__ w_k, const float* __restrict__ w_v, const int32_t* __restrict__ slots,
    int64_t num_slots, float* __restrict__ k_cache, float* __restrict__ v_cache, int num_kv_heads,
    int block_size, int bs_shift, int head_dim, float* __restrict__ rows_out) {
  extern __shared__ float xs[];
  __shared__ float partial[kF32Threads / 64];
  const int t = blockIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float* xr = x + static_cast<int64_t>(t) * hidden;
  float ss = 0.0f;
  for (int i = tid; i < hidden; i += kF32Threads) {
    const float v = xr[i];
    xs[i] = v;
    ss = fmaf(v, v, ss);
  }
#pragma unroll
  for (int mask = 32; mask > 0; mask >>= 1) ss += __shfl_xor(ss, mask, 64);
  if (lane == 0) partial[wave] = ss;
  __syncthreads();
  float total = 0.0f;
#pragma unroll
  for (int w = 0; w < kF32Threads / 64; ++w) total += partial[w];
  const float scale = 1.0f / sqrtf(total / static_cast<float>(hidden) + eps);
  for (int i = tid; i < hidden; i += kF32Threads) xs[i] = xs[i] * scale * w_rms[i];
  __syncthreads();

  const int out_half = num_kv_heads * head_dim;
  const int64_t blk = slot >> bs_shift;
  const int64_t off = slot & (block_size - 1);
  for (int o = wave; o < 2 * out_half; o += kF32Threads / 64) {
    const bool is_v = o >= out_half;
    const int hd = is_v ? o - out_half : o;
    const float* wr = (is_v ? w_v : w_k) + static_cast<int64_t>(hd) * hidden;
    float acc = 0.0f;
    for (int i = lane; i < hidden; i += 64) acc = fmaf(wr[i], xs[i], acc);
#pragma unroll
    for (int mask = 32; mask > 0; mask >>= 1) acc += __shfl_xor(acc, mask, 64);
    if (lane == 0) {
      const int h = hd / head_dim;
      const int d = hd - h * head_dim;
      if (rows_out != nullptr) {
        rows_out[static_cast<int64_t>(t) * 2 * out_half + o] = acc;
      } else {
        float* cache = is_v ? v_cache : k_cache;
        cache[((blk * num_kv_heads + h) * block_size + off) * head_dim + d] = acc;
      }
    }
  }
}

// ---- bf16 skinny path: T <= 64 -------------------------------------------------

constexpr int kSkinnyCols = 16;   // output features per workgroup

struct SkinnyArgs {
  const uint16_t* x;          // [T][H]
  const uint16_t* w_rms;      // [H]
  const uint16_t* w_k;        // [Hkv*D][H]
  const uint16_t* w_v;
  const int32_t* slots;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int32_t num_tokens;
  int32_t hidden;
  int32_t out_half;
  int32_t head_dim;
  int32_t block_size;
  int32_t bs_shift;
  int32_t num_kv_heads;
  int64_t num_slots;
  float inv_hidden;
  float eps;
  float* rows_out;            // fp32 [T][2*Hkv*D] instead of the cache (8-bit cache), or nullptr
};

// kMT tiles of 16 tokens (T <= 16*kMT).  Wavefront w of kSkinnyWaves covers
// hidden columns [w*H/8, (w+1)*H/8); the partial products and sums of
// squares are added in LDS in wavefront order.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyGroup = 4;               // K steps whose loads are issued together

template <int kMT>
__global__ __launch_bounds__(64 * kSkinnyWaves) void kv_append_skinny_kernel(SkinnyArgs a) {
  __shared__ f32x4 s_acc[kSkinnyWaves][kMT][64];
  __shared__ float s_ssq[kSkinnyWaves][kMT * 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * kSkinnyCols;
  const bool is_v = n0 >= a.out_half;           // out_half is a multiple of 64: no tile straddles K and V
  const int col = n0 + (lane & 15);
  const uint16_t* wrow = (is_v ? a.w_v : a.w_k) + static_cast<int64_t>(col - (is_v ? a.out_half : 0)) * a.hidden;
  const int kq = a.hidden / kSkinnyWaves;
  const int k_begin = wave * kq;
  const int kofs = (lane >> 4) * 8;

  // The epilogue's slots (element e = tid + i*512 of the kMT*64*4 outputs),
  // loaded now so that their latency hides behind the products.
  constexpr int kEpi = (kMT * 256 + 64 * kSkinnyWaves - 1) / (64 * kSkinnyWaves);
  int64_t slot_of[kEpi];
#pragma unroll
  for (int i = 0; i < kEpi; ++i) {
    const int e = tid + i * 64 * kSkinnyWaves;
    const int row = (e / 256) * 16 + (((e / 4) & 63) >> 4) * 4 + (e & 3);
    slot_of[i] = e < kMT * 256 && row < a.num_tokens ? static_cast<int64_t>(a.slots[row]) : -1;
  }
  f32x4 acc[kMT];
  float ssq[kMT];
  const uint16_t* xptr[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    ssq[mt] = 0.0f;
    // rows past the last token read the last one: their outputs and sums of
    // squares are never used, so the loads need no select (which would make
    // the compiler wait for them at once)
    const int row = min(mt * 16 + (lane & 15), a.num_tokens - 1);
    xptr[mt] = a.x + static_cast<int64_t>(row) * a.hidden + kofs;
  }
  auto step = [&](const uint4& wb, const uint4& wr, const uint4 (&xv)[kMT]) {
    const uint32_t* wru = reinterpret_cast<const uint32_t*>(&wr);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const uint32_t* xu = reinterpret_cast<const uint32_t*>(&xv[mt]);
      uint4 av;
      uint32_t* au = reinterpret_cast<uint32_t*>(&av);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(xu[e]);
        const float hi = bf16_hi(xu[e]);
        ssq[mt] = fmaf(lo, lo, ssq[mt]);
        ssq[mt] = fmaf(hi, hi, ssq[mt]);
        au[e] = yoco::pack_bf16x2(lo * bf16_lo(wru[e]), hi * bf16_hi(wru[e]));
      }
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                       __builtin_bit_cast(bf16x8, wb), acc[mt], 0, 0, 0);
    }
  };
  // K steps of 32 in groups of kSkinnyGroup: a group's loads are all issued
  // before any is used, so the wavefront waits once per group.
  const int n_steps = kq / 32;
  int st = 0;
  for (; st + kSkinnyGroup <= n_steps; st += kSkinnyGroup) {
    uint4 wb[kSkinnyGroup], wr[kSkinnyGroup], xv[kSkinnyGroup][kMT];
#pragma unroll
    for (int g = 0; g < kSkinnyGroup; ++g) {
      const int k = k_begin + (st + g) * 32;
      wb[g] = *reinterpret_cast<const uint4*>(wrow + k + kofs);
      wr[g] = *reinterpret_cast<const uint4*>(a.w_rms + k + kofs);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) xv[g][mt] = *reinterpret_cast<const uint4*>(xptr[mt] + k);
    }
#pragma unroll
    for (int g = 0; g < kSkinnyGroup; ++g) step(wb[g], wr[g], xv[g]);
  }
  for (; st < n_steps; ++st) {
    const int k = k_begin + st * 32;
    uint4 xv[kMT];
    const uint4 wb = *reinterpret_cast<const uint4*>(wrow + k + kofs);
    const uint4 wr = *reinterpret_cast<const uint4*>(a.w_rms + k + kofs);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) xv[mt] = *reinterpret_cast<const uint4*>(xptr[mt] + k);
    step(wb, wr, xv);
  }
  // Sums of squares: lanes l, l^16, l^32, l^48 hold the same row.
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    float v = ssq[mt];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (lane < 16) s_ssq[wave][mt * 16 + lane] = v;
    s_acc[wave][mt][lane] = acc[mt];
  }
  __syncthreads();

  // Lane l of the MFMA output holds rows 4*(l/16)+0..3 of column l%16.
#pragma unroll
  for (int ei = 0; ei < kEpi; ++ei) {
    const int e = tid + ei * 64 * kSkinnyWaves;
    const int mt = e / 256;
    const int l = (e / 4) & 63;
    const int i = e & 3;
    const int row = mt * 16 + (l >> 4) * 4 + i;
    const int64_t slot = slot_of[ei];
    if (e >= kMT * 256 || row >= a.num_tokens || slot < 0 || slot >= a.num_slots) continue;
    float sum = 0.0f, sq = 0.0f;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves; ++w) {
      sum += s_acc[w][mt][l][i];
      sq += s_ssq[w][mt * 16 + (l >> 4) * 4 + i];
    }
    const float scale = 1.0f / sqrtf(sq * a.inv_hidden + a.eps);
    if (a.rows_out != nullptr) {
      a.rows_out[static_cast<int64_t>(row) * 2 * a.out_half + n0 + (l & 15)] = sum * scale;
      continue;
    }
    const int c = n0 + (l & 15) - (is_v ? a.out_half : 0);
    const int h = c / a.head_dim;
    const int d = c - h * a.head_dim;
    uint16_t* cache = is_v ? a.v_cache : a.k_cache;
    cache[(((slot >> a.bs_shift) * a.num_kv_heads + h) * a.block_size + (slot & (a.block_size - 1))) * a.head_dim + d] =
        f32_to_bf16_rne(sum * scale);
  }
}

// ---- scatter of given rows, optionally quantizing to FP8 E4M3 ---------------------

constexpr int kScatterThreads = 256;
constexpr int kScatterBatchRows = 16;  // rows a quantizing-scatter wavefront loads before reducing any

struct ScatterArgs {
  const void* k_src;          // K rows: token t, KV head h at k_src + t*token_stride + h*D (source elements)
  const void* v_src;
  int64_t token_stride;       // source elements between tokens
  const int32_t* slots;
  void* k_cache;
  void* v_cache;
  float* k_scale;             // [num_blocks][Hkv][bs] (8-bit cache), else nullptr
  float* v_scale;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t bs_shift;
  int64_t num_slots;
};

// One workgroup per token; wavefront w copies the (K or V, KV head) rows
// w, w+4, ... of its token: the row's bytes as they are.
template <bool kSrcF32>
__global__ __launch_bounds__(kScatterThreads) void kv_scatter_kernel(ScatterArgs a) {
  const int t = blockIdx.x;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t blk = slot >> a.bs_shift;
  const int64_t off = slot & (a.block_size - 1);
  const int D = a.head_dim;
  constexpr int kSrcBytes = kSrcF32 ? 4 : 2;
  for (int p = wave; p < 2 * a.num_kv_heads; p += kScatterThreads / 64) {
    const bool is_v = p >= a.num_kv_heads;
    const int h = is_v ? p - a.num_kv_heads : p;
    const char* src = static_cast<const char*>(is_v ? a.v_src : a.k_src) +
                      (static_cast<int64_t>(t) * a.token_stride + static_cast<int64_t>(h) * D) * kSrcBytes;
    const int64_t row = (blk * a.num_kv_heads + h) * a.block_size + off;
    uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(is_v ? a.v_cache : a.k_cache) + row * D * kSrcBytes);
    for (int c = lane; c < D * kSrcBytes / 16; c += 64) dst[c] = reinterpret_cast<const uint4*>(src)[c];
  }
}

// Quantizing scatter to FP8 E4M3. One wavefront per token; its 2*Hkv rows
// (K rows, then V rows) are taken four at a time, a row per 16 lanes: lane l
// works on row 4j + l/16 and holds kVec groups of four consecutive values,
// group v at columns 64v + 4(l%16) .. +3, so each load instruction reads 64
// contiguous values of four rows. Up to kScatterBatchRows rows are loaded
// before any is reduced. The row's largest magnitude is a max over the fp32
// bit patterns (ordered like the magnitudes, and above every finite value for
// inf and NaN); s = max / 448 and code = E4M3(x / s), both divisions in fp32
// (the code mostly found without the second, by e4m3_of_quotient); a row
// holding inf or NaN is stored as NaN codes (its scale is inf or NaN), a row
// of zeros as zero codes with scale 0.
template <bool kSrcF32, int kVec>
__global__ __launch_bounds__(kScatterThreads) void kv_quant_scatter_kernel(ScatterArgs a, int32_t num_tokens) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kScatterThreads / 64) + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  const int64_t slot = a.slots[t];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t blk = slot >> a.bs_shift;
  const int64_t off = slot & (a.block_size - 1);
  constexpr int D = 64 * kVec;
  constexpr int kQuads = kScatterBatchRows / 4;
  const int rows = 2 * a.num_kv_heads;
  const int sub = lane >> 4;         // row within a group of four
  const int col = 4 * (lane & 15);   // first column of this lane's group 0
  for (int r0 = 0; r0 < rows; r0 += 4 * kQuads) {
    float x[kQuads][kVec][4];
#pragma unroll
    for (int j = 0; j < kQuads; ++j) {
      const int p = min(r0 + 4 * j + sub, rows - 1);   // rows past the end reload the last row
      const bool is_v = p >= a.num_kv_heads;
      const int h = is_v ? p - a.num_kv_heads : p;
      const int64_t e0 = static_cast<int64_t>(t) * a.token_stride + static_cast<int64_t>(h) * D + col;
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        if constexpr (kSrcF32) {
          const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(is_v ? a.v_src : a.k_src) + e0 + 64 * v);
          x[j][v][0] = f.x; x[j][v][1] = f.y; x[j][v][2] = f.z; x[j][v][3] = f.w;
        } else {
          const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(is_v ? a.v_src : a.k_src) + e0 + 64 * v);
          x[j][v][0] = __uint_as_float(u.x << 16); x[j][v][1] = __uint_as_float(u.x & 0xffff0000u);
          x[j][v][2] = __uint_as_float(u.y << 16); x[j][v][3] = __uint_as_float(u.y & 0xffff0000u);
        }
      }
    }
    uint32_t mbits[kQuads];
#pragma unroll
    for (int j = 0; j < kQuads; ++j) {
      uint32_t m = 0;
#pragma unroll
      for (int v = 0; v < kVec; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = max(m, __float_as_uint(x[j][v][e]) & 0x7fffffffu);
      mbits[j] = row16_max(m);
    }
#pragma unroll
    for (int j = 0; j < kQuads; ++j) {
      const int p = r0 + 4 * j + sub;
      if (p >= rows) continue;
      const float s = __uint_as_float(mbits[j]) / 448.0f;
      const bool finite = mbits[j] < 0x7f800000u;
      const float r = finite && s > 0.0f ? 1.0f / s : 0.0f;
      const bool is_v = p >= a.num_kv_heads;
      const int h = is_v ? p - a.num_kv_heads : p;
      const int64_t row = (blk * a.num_kv_heads + h) * a.block_size + off;
      uint8_t* dst = static_cast<uint8_t*>(is_v ? a.v_cache : a.k_cache) + row * D + col;
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t code = !finite ? 0x7fu : (s == 0.0f ? 0u : yoco::e4m3_of_quotient(x[j][v][e], s, r));
          packed |= code << (8 * e);
        }
        *reinterpret_cast<uint32_t*>(dst + 64 * v) = packed;
      }
      if ((lane & 15) == 0) (is_v ? a.v_scale : a.k_scale)[row] = s;
    }
  }
}

bool supported_dim(int d) { return d == 64 || d == 128 || d == 256; }

}  // namespace

extern "C" int64_t yoco_kv_append_workspace_size(int32_t dtype, int32_t hidden, int32_t num_kv_heads,
                                                 int32_t head_dim) {
  if (hidden <= 0 || num_kv_heads <= 0 || head_dim <= 0) return -1;
  if (dtype != YOCO_DTYPE_BF16) return 0;
  return static_cast<int64_t>(2) * num_kv_heads * head_dim * hidden * 2;
}

namespace {

// A few tokens whose hidden size the split-K kernel divides go through it;
// the rest (bf16) through the MFMA GEMM.
bool uses_skinny(int32_t num_tokens, int32_t hidden) {
  return num_tokens <= 64 && hidden % (32 * kSkinnyWaves) == 0;
}

// FP8 cache: every path but the MFMA GEMM (which quantizes in its epilogue)
// hands fp32 rows to the quantizing scatter.
bool fp8_needs_rows(int32_t dtype, int32_t num_tokens, int32_t hidden) {
  return dtype == YOCO_DTYPE_F32 || uses_skinny(num_tokens, hidden);
}

int64_t rows_bytes_of(int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim) {
  return static_cast<int64_t>(num_tokens) * 2 * num_kv_heads * head_dim * 4;
}

int32_t scatter_impl(bool src_f32, bool quant, const void* k_src, const void* v_src, int64_t token_stride,
                     int32_t num_tokens, const int32_t* slot_mapping, void* k_cache, void* v_cache, float* k_scale,
                     float* v_scale, int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                     hipStream_t s);

// Validation mode only: the slots checked on a host copy (distinct, inside
// the cache).
int32_t validate_slot_mapping(const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                              hipStream_t s, const char* who) {
  if (!yoco_validation_enabled()) return YOCO_OK;
  std::vector<int32_t> slots;
  bool skip = false;
  const int32_t st = yoco::fetch_indices(slot_mapping, num_tokens, s, slots, skip, who);
  if (st != YOCO_OK || skip) return st;
  return yoco_validate_slots(slots.data(), num_tokens, num_blocks, block_size);
}

int32_t append_impl(int32_t dtype, const void* x, int32_t num_tokens, int32_t hidden, const void* rms_weight,
                    float eps, const void* w_k, const void* w_v, const int32_t* slot_mapping, void* k_cache,
                    void* v_cache, int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                    void* workspace, int64_t workspace_bytes, float* rows_out, int64_t rows_bytes, float* k_scale,
                    float* v_scale, void* stream) {
  // The projection of every scheduled token into its cache slots: caches in
  // `dtype`, or FP8 codes with scales when k_scale != nullptr.  FP8 through
  // the MFMA GEMM quantizes in its epilogue; through the other kernels it goes
  // as fp32 rows [T][2*Hkv*D] into rows_out, then the quantizing scatter.  The
  // fold workspace is the first `fold` bytes of `workspace`.
  using namespace yoco;
  const bool quant = k_scale != nullptr;
  if (dtype != YOCO_DTYPE_F32 && dtype != YOCO_DTYPE_BF16)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_append: unknown dtype %d", dtype);
  if (num_tokens < 0 || hidden <= 0 || num_blocks <= 0 || num_kv_heads <= 0 || workspace_bytes < 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_append: negative or zero size argument");
  if (!std::isfinite(eps) || eps < 0.0f) return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_append: eps must be finite and >= 0");
  if (!supported_dim(head_dim)) return fail(YOCO_ERR_UNSUPPORTED, "kv_append: head_dim %d not in {64,128,256}", head_dim);
  if (!is_pow2(block_size) || block_size > 256)
    return fail(YOCO_ERR_UNSUPPORTED, "kv_append: block_size %d is not a power of two <= 256", block_size);
  if (hidden % 64 != 0) return fail(YOCO_ERR_UNSUPPORTED, "kv_append: hidden %d is not a multiple of 64", hidden);
  if (dtype == YOCO_DTYPE_F32 && hidden > 16384)
    return fail(YOCO_ERR_UNSUPPORTED, "kv_append: fp32 path supports hidden <= 16384");
  const int64_t need = yoco_kv_append_workspace_size(dtype, hidden, num_kv_heads, head_dim) + rows_bytes;
  if (workspace_bytes < need)
    return fail(YOCO_ERR_WORKSPACE_TOO_SMALL, "kv_append: workspace %lld bytes, need %lld",
                (long long)workspace_bytes, (long long)need);
  if (num_tokens == 0) return YOCO_OK;
  if (x == nullptr || rms_weight == nullptr || w_k == nullptr || w_v == nullptr || slot_mapping == nullptr ||
      k_cache == nullptr || v_cache == nullptr || (need > 0 && workspace == nullptr) ||
      (quant && (v_scale == nullptr || (fp8_needs_rows(dtype, num_tokens, hidden) && rows_out == nullptr))))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_append: null pointer");
  if (!aligned16(x) || !aligned16(rms_weight) || !aligned16(w_k) || !aligned16(w_v) || !aligned16(k_cache) ||
      !aligned16(v_cache) || (need > 0 && !aligned16(workspace)))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_append: buffers must be 16-byte aligned");
  const int64_t out_half = static_cast<int64_t>(num_kv_heads) * head_dim;
  auto quantize_rows = [&](int32_t st) {
    if (st != YOCO_OK || !quant) return st;
    return scatter_impl(true, true, rows_out, rows_out + out_half, 2 * out_half, num_tokens, slot_mapping, k_cache,
                        v_cache, k_scale, v_scale, num_blocks, num_kv_heads, block_size, head_dim,
                        static_cast<hipStream_t>(stream));
  };

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t vst = validate_slot_mapping(slot_mapping, num_tokens, num_blocks, block_size, s, "kv_append");
  if (vst != YOCO_OK) return vst;
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  const int bs_shift = ilog2(block_size);
  clear_launch_error();
  if (dtype == YOCO_DTYPE_F32) {
    hipLaunchKernelGGL(kv_append_f32_kernel, dim3(num_tokens), dim3(kF32Threads), hidden * sizeof(float), s,
                       static_cast<const float*>(x), hidden, static_cast<const float*>(rms_weight), eps,
                       static_cast<const float*>(w_k), static_cast<const float*>(w_v), slot_mapping, num_slots,
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), num_kv_heads, block_size,
                       bs_shift, head_dim, quant ? rows_out : nullptr);
    return quantize_rows(launch_result("kv_append"));
  }

  if (uses_skinny(num_tokens, hidden)) {
    SkinnyArgs k;
    k.x = static_cast<const uint16_t*>(x);
    k.w_rms = static_cast<const uint16_t*>(rms_weight);
    k.w_k = static_cast<const uint16_t*>(w_k);
    k.w_v = static_cast<const uint16_t*>(w_v);
    k.slots = slot_mapping;
    k.k_cache = static_cast<uint16_t*>(k_cache);
    k.v_cache = static_cast<uint16_t*>(v_cache);
    k.num_tokens = num_tokens;
    k.hidden = hidden;
    k.out_half = static_cast<int32_t>(out_half);
    k.head_dim = head_dim;
    k.block_size = block_size;
    k.bs_shift = bs_shift;
    k.num_kv_heads = num_kv_heads;
    k.num_slots = num_slots;
    k.inv_hidden = 1.0f / static_cast<float>(hidden);
    k.eps = eps;
    k.rows_out = quant ? rows_out : nullptr;
    const dim3 grid(static_cast<uint32_t>(2 * out_half / kSkinnyCols));
    const dim3 block(64 * kSkinnyWaves);
    if (num_tokens <= 16) {
      hipLaunchKernelGGL(kv_append_skinny_kernel<1>, grid, block, 0, s, k);
    } else if (num_tokens <= 32) {
      hipLaunchKernelGGL(kv_append_skinny_kernel<2>, grid, block, 0, s, k);
    } else {
      hipLaunchKernelGGL(kv_append_skinny_kernel<4>, grid, block, 0, s, k);
    }
    return quantize_rows(launch_result("kv_append"));
  }
  const int64_t half_chunks = out_half * hidden / 8;
  const int64_t fold_blocks = ceil_div(2 * half_chunks, 256);
  hipLaunchKernelGGL(fold_rms_weight_kernel, dim3(static_cast<uint32_t>(fold_blocks)), dim3(256), 0, s,
                     static_cast<const uint4*>(w_k), static_cast<const uint4*>(w_v),
                     static_cast<const uint4*>(rms_weight), static_cast<uint4*>(workspace), half_chunks, hidden / 8);

  AppendArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(workspace);
  a.slots = slot_mapping;
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.num_tokens = num_tokens;
  a.hidden = hidden;
  a.out_half = static_cast<int32_t>(out_half);
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.bs_shift = bs_shift;
  a.num_kv_heads = num_kv_heads;
  a.num_slots = num_slots;
  a.inv_hidden = 1.0f / static_cast<float>(hidden);
  a.eps = eps;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.n_tiles = static_cast<int32_t>(ceil_div(2 * out_half, kBN));
  const int64_t tiles = ceil_div(num_tokens, kBM) * a.n_tiles;
  if (tiles > 0x7fffffff / 2) return fail(YOCO_ERR_UNSUPPORTED, "kv_append: %lld GEMM tiles", (long long)tiles);
  a.num_tiles = static_cast<int32_t>(tiles);
  a.tiles_per_xcd = static_cast<int32_t>(ceil_div(tiles, 8));
  const dim3 grid(static_cast<uint32_t>(8 * a.tiles_per_xcd)), block(kGemmThreads);
  if (!quant) hipLaunchKernelGGL(kv_append_mfma_kernel<0>, grid, block, 0, s, a);
  else if (head_dim == 64) hipLaunchKernelGGL(kv_append_mfma_kernel<64>, grid, block, 0, s, a);
  else if (head_dim == 128) hipLaunchKernelGGL(kv_append_mfma_kernel<128>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(kv_append_mfma_kernel<256>, grid, block, 0, s, a);
  return launch_result("kv_append");
}

bool is_f8(int32_t dtype) { return dtype == YOCO_DTYPE_FP8_E4M3; }

// Launch the scatter of rows [T][Hkv][D] (token stride given) into the cache.
int32_t scatter_impl(bool src_f32, bool quant, const void* k_src, const void* v_src, int64_t token_stride,
                     int32_t num_tokens, const int32_t* slot_mapping, void* k_cache, void* v_cache, float* k_scale,
                     float* v_scale, int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                     hipStream_t s) {
  ScatterArgs a;
  a.k_src = k_src;
  a.v_src = v_src;
  a.token_stride = token_stride;
  a.slots = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.bs_shift = yoco::ilog2(block_size);
  a.num_slots = static_cast<int64_t>(num_blocks) * block_size;
  const dim3 block(kScatterThreads);
  if (quant) {
    constexpr int kTokensPerGroup = kScatterThreads / 64;
    const dim3 grid(static_cast<uint32_t>((num_tokens + kTokensPerGroup - 1) / kTokensPerGroup));
    const int vec = head_dim / 64;
    if (src_f32) {
      if (vec == 4) hipLaunchKernelGGL((kv_quant_scatter_kernel<true, 4>), grid, block, 0, s, a, num_tokens);
      else if (vec == 2) hipLaunchKernelGGL((kv_quant_scatter_kernel<true, 2>), grid, block, 0, s, a, num_tokens);
      else hipLaunchKernelGGL((kv_quant_scatter_kernel<true, 1>), grid, block, 0, s, a, num_tokens);
    } else {
      if (vec == 4) hipLaunchKernelGGL((kv_quant_scatter_kernel<false, 4>), grid, block, 0, s, a, num_tokens);
      else if (vec == 2) hipLaunchKernelGGL((kv_quant_scatter_kernel<false, 2>), grid, block, 0, s, a, num_tokens);
      else hipLaunchKernelGGL((kv_quant_scatter_kernel<false, 1>), grid, block, 0, s, a, num_tokens);
    }
  } else {
    const dim3 grid(static_cast<uint32_t>(num_tokens));
    if (src_f32) hipLaunchKernelGGL((kv_scatter_kernel<true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((kv_scatter_kernel<false>), grid, block, 0, s, a);
  }
  return yoco::launch_result("kv_scatter");
}

}  // namespace

extern "C" int32_t yoco_kv_append(int32_t dtype, const void* x, int32_t num_tokens, int32_t hidden,
                                  const void* rms_weight, float eps, const void* w_k, const void* w_v,
                                  const int32_t* slot_mapping, void* k_cache, void* v_cache, int32_t num_blocks,
                                  int32_t num_kv_heads, int32_t block_size, int32_t head_dim, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
  return append_impl(dtype, x, num_tokens, hidden, rms_weight, eps, w_k, w_v, slot_mapping, k_cache, v_cache,
                     num_blocks, num_kv_heads, block_size, head_dim, workspace, workspace_bytes, nullptr, 0, nullptr,
                     nullptr, stream);
}

extern "C" int64_t yoco_kv_append_fp8_workspace_size(int32_t dtype, int32_t num_tokens, int32_t hidden,
                                                     int32_t num_kv_heads, int32_t head_dim) {
  if (num_tokens < 0) return -1;
  const int64_t fold = yoco_kv_append_workspace_size(dtype, hidden, num_kv_heads, head_dim);
  if (fold < 0) return -1;
  return yoco::round_up(fold, 256) +
         (fp8_needs_rows(dtype, num_tokens, hidden) ? rows_bytes_of(num_tokens, num_kv_heads, head_dim) : 0);
}

extern "C" int32_t yoco_kv_append_fp8(int32_t dtype, const void* x, int32_t num_tokens, int32_t hidden,
                                      const void* rms_weight, float eps, const void* w_k, const void* w_v,
                                      const int32_t* slot_mapping, void* k_cache, void* v_cache, float* k_scale,
                                      float* v_scale, int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                                      int32_t head_dim, void* workspace, int64_t workspace_bytes, void* stream) {
  using namespace yoco;
  if (num_tokens < 0 || hidden <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_append_fp8: negative or zero size argument");
  const int64_t fold = yoco_kv_append_workspace_size(dtype, hidden, num_kv_heads, head_dim);
  const int64_t need = yoco_kv_append_fp8_workspace_size(dtype, num_tokens, hidden, num_kv_heads, head_dim);
  if (fold < 0 || need < 0) return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_append_fp8: bad dtype or shape");
  if (workspace_bytes < need)
    return fail(YOCO_ERR_WORKSPACE_TOO_SMALL, "kv_append_fp8: workspace %lld bytes, need %lld",
                (long long)workspace_bytes, (long long)need);
  if (num_tokens > 0 && (k_cache == nullptr || v_cache == nullptr || k_scale == nullptr || v_scale == nullptr ||
                         workspace == nullptr))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_append_fp8: null pointer");
  if (num_tokens > 0 && (!aligned16(workspace) || !aligned16(k_cache) || !aligned16(v_cache) ||
                         (reinterpret_cast<uintptr_t>(k_scale) & 3) != 0 ||
                         (reinterpret_cast<uintptr_t>(v_scale) & 3) != 0))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_append_fp8: workspace and caches must be 16-byte, scales 4-byte aligned");
  const bool with_rows = num_tokens > 0 && fp8_needs_rows(dtype, num_tokens, hidden);
  float* rows = with_rows ? reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up(fold, 256)) : nullptr;
  const int64_t rb = with_rows ? rows_bytes_of(num_tokens, num_kv_heads, head_dim) : 0;
  return append_impl(dtype, x, num_tokens, hidden, rms_weight, eps, w_k, w_v, slot_mapping, k_cache, v_cache,
                     num_blocks, num_kv_heads, block_size, head_dim, workspace, workspace_bytes - rb, rows, 0, k_scale,
                     v_scale, stream);
}

extern "C" int32_t yoco_kv_scatter(int32_t src_dtype, const void* k_rows, const void* v_rows, int32_t num_tokens,
                                   const int32_t* slot_mapping, int32_t cache_dtype, void* k_cache, void* v_cache,
                                   float* k_scale, float* v_scale, int32_t num_blocks, int32_t num_kv_heads,
                                   int32_t block_size, int32_t head_dim, void* stream) {
  using namespace yoco;
  if (src_dtype != YOCO_DTYPE_F32 && src_dtype != YOCO_DTYPE_BF16)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_scatter: unknown source dtype %d", src_dtype);
  const bool quant = is_f8(cache_dtype);
  if (!quant && cache_dtype != src_dtype)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_scatter: cache dtype %d must be the source dtype or FP8", cache_dtype);
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_scatter: negative or zero size argument");
  if (!supported_dim(head_dim)) return fail(YOCO_ERR_UNSUPPORTED, "kv_scatter: head_dim %d not in {64,128,256}", head_dim);
  if (!is_pow2(block_size) || block_size > 256)
    return fail(YOCO_ERR_UNSUPPORTED, "kv_scatter: block_size %d is not a power of two <= 256", block_size);
  if (quant != (k_scale != nullptr) || quant != (v_scale != nullptr))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_scatter: scales are required for, and only for, an FP8 cache");
  if (num_tokens == 0) return YOCO_OK;
  if (k_rows == nullptr || v_rows == nullptr || slot_mapping == nullptr || k_cache == nullptr || v_cache == nullptr)
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_scatter: null pointer");
  if (!aligned16(k_rows) || !aligned16(v_rows) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(YOCO_ERR_INVALID_ARGUMENT, "kv_scatter: rows and caches must be 16-byte aligned");
  const int32_t vst = validate_slot_mapping(slot_mapping, num_tokens, num_blocks, block_size,
                                            static_cast<hipStream_t>(stream), "kv_scatter");
  if (vst != YOCO_OK) return vst;
  clear_launch_error();
  return scatter_impl(src_dtype == YOCO_DTYPE_F32, quant, k_rows, v_rows,
                      static_cast<int64_t>(num_kv_heads) * head_dim, num_tokens, slot_mapping, k_cache, v_cache,
                      k_scale, v_scale, num_blocks, num_kv_heads, block_size, head_dim,
                      static_cast<hipStream_t>(stream));
}
