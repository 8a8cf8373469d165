// Matrix-core variant of the cross-attention kernel (included by
// cross_attn_kernels.h, after the VALU kernel whose helpers it uses).
//
// When the work per K^/V^ byte grows -- an 8-bit cache (twice the rows per
// byte) or several query rows per request (up to 16 query vectors per KV
// group) -- the VALU kernel runs out of vector throughput, while q.k and p.v
// are then small dense contractions.  Here a work item's query vectors
// (G heads x its query rows, padded to 16) sit in registers as an MFMA
// operand, and each wavefront streams 16-key tiles of its item:
//
//   S^T[16 keys][16 q] = K[16 keys][D] . Q^T[D][16 q]
//       v_mfma_f32_16x16x32_bf16 over head_dim; K rows are loaded from the
//       paged cache directly in the A-operand layout (lane l: key l%16, eight
//       head_dim elements), FP8 rows widened exactly to bf16 in registers.
//   online softmax: lane l owns query l%16 and four keys of each tile; the
//       running max of a query is shared by its four lanes (two shuffles).
//   O^T[D][16 q] += V^T[D][16 keys] . P^T[16 keys][16 q]
//       v_mfma_f32_16x16x16_bf16; V goes through a per-wavefront LDS tile
//       (written row-major, read as the transposed A operand with one
//       ds_read_b64_tr_b16 per operand), P^T is exactly the lane's own
//       softmax weights.  P is split
//       into bf16 high and low parts (two products), so the weights keep ~17
//       bits; K, V (bf16 or widened FP8) and q are exact bf16 values, and all
//       sums are fp32.  Each lane's O^T column belongs to its own query, so
//       rescaling on a new maximum stays lane-local.
//
// At head_dim 256 several wavefronts share each key tile, each with a slice
// of head_dim (bf16: four slices, the scores summed through LDS; FP8: two,
// each computing the whole scores), which keeps two wavefronts per SIMD; a
// bf16 cache at head_dim 256 takes this kernel also for one query row.
//
// The schedule, work items, partials, item pipeline and the merge kernel are
// those of the VALU kernel: the next item is fetched before the current one's
// last iteration, whose row request is already the next item's first tile.

#pragma once

namespace yoco_attn {

typedef __bf16 mfma_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 mfma_bf16x4 __attribute__((ext_vector_type(4)));
typedef float mfma_f32x4 __attribute__((ext_vector_type(4)));

template <int kT, int D>
struct MfmaLayout {
  static_assert(kT == kBF16 || kT == kFP8, "bf16 or FP8 cache");
  static constexpr int kEb = kT == kFP8 ? 1 : 2;                       // cache element bytes
  static constexpr int kRowBytes = D * kEb;
  // keys per wavefront iteration: about 8 KB of K^/V^ (bf16) or 4 KB (FP8,
  // which keeps two wavefronts per SIMD in registers), at least one tile
  static constexpr int kBudget = kT == kFP8 ? 4096 : 8192;
  // head_dim 256, bf16: the four wavefronts of a workgroup stream the same
  // keys, each with one 64-column slice of head_dim: its part of every score
  // (the four parts summed through LDS, one barrier per iteration) and its
  // 64 rows of O^T.  A wavefront then holds a quarter of the rows and
  // accumulators, so two fit per SIMD, and no K row is read twice
  // (decode64 with 4 rows per request: 138 -> 116 us per layer).
  // head_dim 256, FP8: wavefront pairs stream the same keys, each computing
  // the whole scores and its half of O^T (two per SIMD as well; the split
  // into four, with 16 KB of rows per barrier, was slower: 74 -> 91 us).
  static constexpr bool kSplit = D == 256 && kT == kBF16;
  static constexpr bool kPair = D == 256 && kT == kFP8;
  static constexpr int kSlices = kSplit ? 4 : kPair ? 2 : 1;          // wavefronts sharing one key tile
  static constexpr int kNK = kSplit ? 32
                           : kBudget / (2 * kRowBytes) < 16 ? 16
                           : (kBudget / (2 * kRowBytes) > 64 ? 64 : kBudget / (2 * kRowBytes));
  static constexpr int kNT = kNK / 16;                                 // 16-key tiles per iteration
  static constexpr int kDW = D / kSlices;                              // head_dim columns of a wavefront's O^T
  static constexpr int kKD = kSplit ? kDW : D;                         // head_dim columns of its scores
  static constexpr int kKS = kKD / 32;                                 // MFMA k-steps over those columns
  static constexpr int kKL = kT == kFP8 ? kKD / 64 : kKD / 32;         // 16-byte K loads per tile per lane
  static constexpr int kVRowBytes = kDW * kEb;                         // bytes of a V row a wavefront loads
  static constexpr int kVC = kNK * kVRowBytes / 16 / 64;               // 16-byte V chunks per lane per iteration
  static constexpr int kChunksPerRow = kVRowBytes / 16;
  // bf16 elements per LDS row of a V tile: the row stride is 8 banks mod 32,
  // so the four rows of one transposed read hit disjoint banks
  static constexpr int kVStride = kDW + 16;
  static_assert(kVC >= 1 && kNK * kVRowBytes % (16 * 64) == 0, "V tile split");
};

// Head_dim offset of the eight k-elements that lane group gi (= lane/16)
// holds at MFMA k-step ks.  bf16: one 16-byte load per step; FP8: one
// 16-byte load covers two steps.  A and B operands use the same map.
template <int kT>
__device__ __forceinline__ int mfma_d_of(int gi, int ks) {
  if constexpr (kT == kFP8) {
    return 64 * (ks >> 1) + 16 * gi + 8 * (ks & 1);
  } else {
    return 32 * ks + 8 * gi;
  }
}

template <int kT, int D, int VG, bool kVar>
struct MfmaSmem {
  using ML = MfmaLayout<kT, D>;
  int32_t len[kMaxQueueSeqs];
  int32_t qs[kVar ? kMaxQueueSeqs + 1 : 1];
  int32_t pref[kMaxQueueSeqs + 1];
  int32_t pref2[kMaxQueueSeqs + 1];
  int32_t wsum[2 * kWaves];
  uint32_t next;
  int32_t blocks[kMaxSliceBlocks];
  union __attribute__((aligned(16))) {
    uint16_t q[16][D + 8];       // the item's query vectors, bf16, rows past VG zero (read into registers)
    // head_dim 256: each wavefront's part of the iteration's scores, in its
    // MFMA output layout, by iteration parity (written once the queries are
    // in registers)
    mfma_f32x4 sc[ML::kSplit ? 2 : 1][ML::kSplit ? kWaves : 1][ML::kSplit ? ML::kNT : 1][64];
  };
  float ml[kWaves][VG][2];
  union __attribute__((aligned(16))) {
    uint16_t vt[kWaves][ML::kNK][ML::kVStride];     // per-wavefront V tile, bf16 row-major
    float acc[kWaves][VG][ML::kDW];                 // per-wavefront outputs for the final combine
  } u;
};

template <int kT, int D, int G, int QPI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void cross_attn_mfma_kernel(AttnArgs a) {
  using ML = MfmaLayout<kT, D>;
  constexpr bool kVar = QPI > 0;
  constexpr bool kF8 = kT == kFP8;
  constexpr int kQ = kVar ? QPI : 1;
  constexpr int VG = G * kQ;
  static_assert(VG <= 16, "at most 16 query vectors per item");
  constexpr int kNK = ML::kNK, kNT = ML::kNT, kKS = ML::kKS, kKL = ML::kKL, kVC = ML::kVC;
  constexpr int kEb = ML::kEb;
  constexpr bool kSplit = ML::kSplit;
  constexpr int kDW = ML::kDW;
  constexpr int kDT = kDW / 16;                     // 16-row tiles of this wavefront's O^T
  constexpr int kSlices = ML::kSlices;              // wavefronts sharing one key tile
  constexpr int kGroups = kWaves / kSlices;         // wavefront groups taking every kGroups-th iteration
  using Smem = MfmaSmem<kT, D, VG, kVar>;
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;                        // key (A/S rows) or query (B/S columns) within a tile
  const int gi = lane >> 4;                         // lane group
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int slice = wave_u % kSlices;               // this wavefront's head_dim slice of O^T
  const int group_u = wave_u / kSlices;
  const int kslice = kSplit ? slice * kDW : 0;      // first head_dim column of its scores
  const bool reverse = (a.flags & YOCO_FLAG_REVERSE_ORDER) != 0;
  const int R = a.num_seqs;
  uint32_t* fetch_ctr = a.queue;
  uint32_t* done_ctr = a.queue + kQueueLineWords;

  auto qlen_of = [&](int r) -> int {
    if constexpr (kVar) {
      return min(max(sm.qs[r + 1] - sm.qs[r], 0), a.max_qlen);
    } else {
      return 1;
    }
  };

  // ---- schedule: per-request item counts and their prefixes (as in the VALU kernel)
  for (int i = tid; i < R; i += kThreads) {
    const int n = a.seq_lens[i];
    sm.len[i] = n < 0 ? 0 : (n > a.len_cap ? a.len_cap : n);
  }
  if constexpr (kVar) {
    for (int i = tid; i <= R; i += kThreads) sm.qs[i] = min(max(a.qsl[i], 0), a.num_rows);
  }
  __syncthreads();
  uint32_t total = 0, total_big = 0;
  {
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

  auto item_at = [&](uint32_t k) -> Item {
    if (k >= total) return make_item(false, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, a.bs_shift);
    // reversed as a whole without tail pieces, else within the big and
    // within the small items (the pieces stay last)
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

  auto valid_block = [&](int b) { return static_cast<unsigned>(b) < static_cast<unsigned>(a.num_blocks) ? b : -1; };

  // ---- registers of one iteration: this wavefront's K (A-operand layout), V
  // (row chunks for the LDS tile), the validity of its score keys and (FP8)
  // their scales.
  //
  // A wavefront iteration covers kNK keys from a 16-aligned position, so with
  // block_size >= 16 every 16-key tile lies inside one cache block: one
  // block-table entry per tile gives a wave-uniform 64-bit row base, and lanes
  // add 32-bit offsets.  Keys before the item's start or past its end, and
  // tiles in an out-of-range block (which read block 0), are masked.  A tile
  // wholly past the item's end reads the 16-aligned tile that holds the
  // item's first key instead (never the item's start itself: with a window
  // the start is rarely 16-aligned, and 16 rows from it could cross the end
  // of its block -- and of the cache, for the last block's last KV head).
  struct Rows {
    uint4 k[kNT][kKL];
    uint4 v[kVC];
    uint32_t vmask;                // bit c: V chunk c's key is an item row in a valid block (else zeroed)
    uint32_t tmask;                // bit t: tile t is a valid block
    int base;                      // logical position of the iteration's first key
    float4 ks[kNT];                // FP8: scales of this lane's score keys base + 16t + 4gi + 0..3
    float4 vs[kNT];
  };

  const int off_mask = a.block_size - 1;
  // Block ids of this wavefront's first tiles of the next item (from the
  // block table while that item's slice is not in LDS yet).
  int32_t st_nb[kNT];
  // Rows of an iteration starting at `base` of the item with key range
  // [start, end), first slice entry first_blk and KV head g; block ids from
  // the LDS slice, or (next) from st_nb.  Both sources are read, so there is
  // no branch around the loads.
  auto load_rows = [&](Rows& rs, int start, int end, int first_blk, int g, int base, bool next) {
    rs.base = base;
    rs.tmask = 0u;
    int64_t tile_row[kNT];         // cache row (block*Hkv + g)*bs + slot of each tile's first key
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      const int p0 = base + 16 * t;
      const int in = p0 < end ? p0 : (start & ~15);
      const int lds_blk = sm.blocks[next ? 0 : (in >> a.bs_shift) - first_blk];
      const int blk = uniform(next ? st_nb[t] : lds_blk);
      const bool ok = blk >= 0;
      rs.tmask |= ok ? (1u << t) : 0u;
      tile_row[t] = (static_cast<int64_t>(ok ? blk : 0) * a.num_kv_heads + g) * a.block_size + (in & off_mask);
      const char* kt = static_cast<const char*>(a.k) + tile_row[t] * ML::kRowBytes;
#pragma unroll
      for (int c = 0; c < kKL; ++c) {
        const int d = kslice + (kF8 ? 64 * c + 16 * gi : 32 * c + 8 * gi);
        rs.k[t][c] = *reinterpret_cast<const uint4*>(kt + l16 * ML::kRowBytes + d * kEb);
      }
      if constexpr (kF8) {
        rs.ks[t] = *reinterpret_cast<const float4*>(a.k_scale + tile_row[t] + 4 * gi);
        rs.vs[t] = *reinterpret_cast<const float4*>(a.v_scale + tile_row[t] + 4 * gi);
      }
    }
    rs.vmask = 0u;
#pragma unroll
    for (int c = 0; c < kVC; ++c) {
      // the 64 chunks of one load instruction belong to 64 / kChunksPerRow <= 16
      // consecutive keys of one tile; a wavefront loads its slice of each row
      constexpr int kKeysPerInst = 64 / ML::kChunksPerRow;
      const int t = (c * kKeysPerInst) / 16;
      const int chunk = lane + 64 * c;
      const int key = chunk / ML::kChunksPerRow;
      const int cb = (chunk - key * ML::kChunksPerRow) * 16 + slice * ML::kVRowBytes;
      const int j = base + key;
      rs.vmask |= ((rs.tmask >> t & 1u) != 0u && j >= start && j < end ? 1u : 0u) << c;
      rs.v[c] = yoco::load_stream(static_cast<const char*>(a.v) + (tile_row[t] + (key - 16 * t)) * ML::kRowBytes + cb);
    }
  };

  // Query operand (B of S^T): query l16's eight elements at each k-step.
  mfma_bf16x8 qop[kKS];
  float m_run = kInitMax, l_run = 0.0f;
  mfma_f32x4 oacc[kDT];
  // per-key tests as one unsigned compare each: key j is in [lo, lo + len)
  // iff unsigned(j - lo) < unsigned(len)
  int item_lo = 0;                                  // the item's range [item_lo, item_lo + item_len)
  uint32_t item_len = 0u;
  int vis_lo = 0;                                   // keys this lane's query sees: [vis_lo, vis_lo + vis_len)
  uint32_t vis_len = 0u;                            // (0 when the lane's column holds no query)

  auto compute = [&](const Rows& rs, const int buf) {
    uint16_t(*vt)[ML::kVStride] = sm.u.vt[wave];
    // the previous iteration's reads of this wavefront's tile come first
    __builtin_amdgcn_wave_barrier();
    // V chunks -> this wavefront's LDS tile as bf16 (masked rows zero)
#pragma unroll
    for (int c = 0; c < kVC; ++c) {
      const int chunk = lane + 64 * c;
      const int key = chunk / ML::kChunksPerRow;
      const int e0 = (chunk - key * ML::kChunksPerRow) * (16 / kEb);  // first element of the chunk
      // masked rows become zero by an AND (a select here compiles to a branch
      // and register copies)
      const uint32_t keep = 0u - ((rs.vmask >> c) & 1u);
      const uint4 vc = make_uint4(rs.v[c].x & keep, rs.v[c].y & keep, rs.v[c].z & keep, rs.v[c].w & keep);
      if constexpr (kF8) {
        uint4 lo8, hi8;
        fp8_to_bf16(vc, lo8, hi8);
        *reinterpret_cast<uint2*>(&vt[key][e0]) = make_uint2(lo8.x, lo8.y);
        *reinterpret_cast<uint2*>(&vt[key][e0 + 4]) = make_uint2(lo8.z, lo8.w);
        *reinterpret_cast<uint2*>(&vt[key][e0 + 8]) = make_uint2(hi8.x, hi8.y);
        *reinterpret_cast<uint2*>(&vt[key][e0 + 12]) = make_uint2(hi8.z, hi8.w);
      } else {
        *reinterpret_cast<uint2*>(&vt[key][e0]) = make_uint2(vc.x, vc.y);
        *reinterpret_cast<uint2*>(&vt[key][e0 + 4]) = make_uint2(vc.z, vc.w);
      }
    }
    // the tile's rows come from other lanes of this wavefront: wait for the
    // LDS writes before reading them back
    __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    // S^T tiles (head_dim 256: this wavefront's slice of every score, the
    // four slices then summed in wavefront order, the same sum in every
    // wavefront)
    mfma_f32x4 sacc[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      mfma_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < kKL; ++c) {
        if constexpr (kF8) {
          uint4 lo8, hi8;
          fp8_to_bf16(rs.k[t][c], lo8, hi8);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mfma_bf16x8, lo8), qop[2 * c], acc, 0, 0,
                                                         0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mfma_bf16x8, hi8), qop[2 * c + 1], acc,
                                                         0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mfma_bf16x8, rs.k[t][c]), qop[c], acc,
                                                         0, 0, 0);
        }
      }
      sacc[t] = acc;
    }
    if constexpr (kSplit) {
#pragma unroll
      for (int t = 0; t < kNT; ++t) sm.sc[buf][wave][t][lane] = sacc[t];
      __syncthreads();
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        mfma_f32x4 sum = sm.sc[buf][0][t][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) sum += sm.sc[buf][w][t][lane];
        sacc[t] = sum;
      }
    }
    float s[kNT][4];
    bool inrange[kNT][4];          // the key is a row of the item (its V and scale are real)
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      const mfma_f32x4 acc = sacc[t];
      const bool tile_ok = (rs.tmask >> t & 1u) != 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = rs.base + 16 * t + 4 * gi + e;
        inrange[t][e] = tile_ok && static_cast<uint32_t>(j - item_lo) < item_len;
        const bool ok = tile_ok && static_cast<uint32_t>(j - vis_lo) < vis_len;
        float sc = a.scale_log2;
        if constexpr (kF8) sc *= e == 0 ? rs.ks[t].x : e == 1 ? rs.ks[t].y : e == 2 ? rs.ks[t].z : rs.ks[t].w;
        s[t][e] = ok ? acc[e] * sc : -INFINITY;
      }
    }
    // online softmax of this lane's query: the iteration's max over its four
    // lanes, lazy rescale, weights
    float tmax = s[0][0];
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, s[t][e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (tmax > m_run + kLazyMaxSlack) {
      const float corr = fast_exp2(m_run - tmax);
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) oacc[dt] *= corr;
      m_run = tmax;
    }
    mfma_bf16x4 p_hi[kNT], p_lo[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(s[t][e] - m_run);
        l_run += p;
        if constexpr (kF8) {
          const float vsc = e == 0 ? rs.vs[t].x : e == 1 ? rs.vs[t].y : e == 2 ? rs.vs[t].z : rs.vs[t].w;
          pv[e] = inrange[t][e] ? p * vsc : 0.0f;
        } else {
          pv[e] = p;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 h = static_cast<__bf16>(pv[e]);
        p_hi[t][e] = h;
        p_lo[t][e] = static_cast<__bf16>(pv[e] - static_cast<float>(h));
      }
    }
    // O^T += V^T P^T per 16-row tile of head_dim
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        // A operand: lane (d = 16dt + l16, keys 16t + 4gi + 0..3).  The
        // transposed LDS read gives lane i of a 16-lane group element i % 4
        // of the 8 bytes that lane 4j + i/4 addressed, in slot j; so lane
        // l16 addresses key 16t + 4gi + l16/4, elements 16dt + 4(l16 % 4)..+3.
        typedef short v4s __attribute__((ext_vector_type(4)));
        const v4s raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (v4s __attribute__((address_space(3)))*)(&vt[16 * t + 4 * gi + (l16 >> 2)][16 * dt + 4 * (l16 & 3)]));
        const mfma_bf16x4 va = __builtin_bit_cast(mfma_bf16x4, raw);
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, p_hi[t], oacc[dt], 0, 0, 0);
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, p_lo[t], oacc[dt], 0, 0, 0);
      }
    }
  };

  // ---- an item's block-table slice and query vectors (and the block ids of
  // this wavefront's first tiles): loaded into registers while the previous
  // item streams, stored to LDS during its hand-over.  Indices are clamped
  // into range so the loads need no branch; what they stand in for is masked
  // at the store.
  constexpr int kTblPer = kMaxSliceBlocks / kThreads;
  constexpr int kQChunks = 16 * (D / 8);                 // 16-byte chunks of the 16 query vectors
  constexpr int kQPer = (kQChunks + kThreads - 1) / kThreads;
  static_assert(kMaxSliceBlocks % kThreads == 0, "slice staging");
  int32_t st_tbl[kTblPer];
  uint4 st_q[kQPer];
  auto stage_load = [&](const Item& it) {
    if (it.num_blk > 0) {
      const int32_t* row_table = a.block_table + static_cast<int64_t>(it.r) * a.max_blocks;
      const int32_t* table = row_table + it.first_blk;
#pragma unroll
      for (int k = 0; k < kTblPer; ++k) st_tbl[k] = table[min(tid + kThreads * k, it.num_blk - 1)];
      // the tiles of this wavefront's first iteration (as load_rows places them)
      const int base = (it.start & ~15) + group_u * kNK;
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const int p0 = base + 16 * t;
        const int in = p0 < it.end ? p0 : (it.start & ~15);
        st_nb[t] = valid_block(row_table[in >> a.bs_shift]);
      }
    }
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int i = min(tid + kThreads * k, kQChunks - 1);
      const int v = min(i / (D / 8), VG - 1);
      const int c = i % (D / 8);
      const int qi = v / G;
      const int h = v - qi * G;
      const int qrow = kVar ? it.row0 + min(qi, max(it.nq - 1, 0)) : it.r;
      st_q[k] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                ((static_cast<int64_t>(qrow) * a.num_q_heads + it.g * G + h) * D +
                                                 c * 8) * 2);
    }
  };
  auto stage_store = [&](const Item& it) {
#pragma unroll
    for (int k = 0; k < kTblPer; ++k) {
      const int i = tid + kThreads * k;
      if (i < it.num_blk) sm.blocks[i] = valid_block(st_tbl[k]);
    }
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int i = tid + kThreads * k;
      if (i < kQChunks) {
        const int v = i / (D / 8);
        *reinterpret_cast<uint4*>(&sm.q[v][(i % (D / 8)) * 8]) = v < VG ? st_q[k] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  // ---- items, pipelined as in the VALU kernel: the next item is known
  // before the current one's last iteration (fetched at the start of a short
  // item, or three rounds before the end of a longer one), that iteration
  // requests this wavefront's first rows of it, and its slice and queries go
  // to LDS while the finished item is combined.  A wavefront runs its
  // iterations in pairs (ra, then rb; an odd count ends with a masked
  // stand-in in rb), so the next item's first rows always land in ra and
  // only one register set lives across the hand-over.
  Item cur = item_at(blockIdx.x);
  Item nxt = make_item(false, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, a.bs_shift);
  if (cur.valid) {
    stage_load(cur);
    stage_store(cur);
  }
  __syncthreads();
  Rows ra, rb;                                      // ra: this wavefront's first rows of `cur`
  if (cur.valid && cur.num_blk > 0)
    load_rows(ra, cur.start, cur.end, cur.first_blk, cur.g, (cur.start & ~15) + group_u * kNK, false);
  while (cur.valid) {
    const int base0 = cur.start & ~15;              // iterations start 16-aligned
    const int num_iters = cur.num_blk > 0 ? (cur.end - base0 + kNK - 1) / kNK : 0;
    const int rounds = num_iters / kGroups;         // iterations every wavefront group has
    // with a workgroup for every item no fetch can return one: none is made
    const bool fetch = gridDim.x < total;
    const bool late = fetch && rounds >= 3;
    if (fetch && !late) {
      if (tid == 0) sm.next = gridDim.x + atomicAdd(fetch_ctr, 1u);
      __syncthreads();
      nxt = item_at(static_cast<uint32_t>(uniform(static_cast<int>(sm.next))));
      stage_load(nxt);
    }
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
    // Rows of iteration i of `cur`; past its end (second of a pair) this
    // wavefront's first rows of `nxt` when that has rows, else a masked
    // stand-in.
    auto load_step = [&](Rows& rs, int i, bool may_next) {
      const bool next = may_next && i >= num_iters && nxt.valid && nxt.num_blk > 0;
      load_rows(rs, next ? nxt.start : cur.start, next ? nxt.end : cur.end, next ? nxt.first_blk : cur.first_blk,
                next ? nxt.g : cur.g, next ? (nxt.start & ~15) + group_u * kNK : base0 + i * kNK, next);
    };

    if (cur.num_blk > 0) {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        qop[ks] = *reinterpret_cast<const mfma_bf16x8*>(&sm.q[l16][kslice + mfma_d_of<kT>(gi, ks)]);
      if constexpr (kSplit) __syncthreads();        // the scores' LDS overlays the queries
      // this lane's query column: vector l16 = query row l16 / G, head l16 % G
      {
        const int qi = l16 / G;
        const bool qlive = l16 < VG && qi < cur.nq;
        const int p = cur.pbase + qi;
        item_lo = cur.start;
        item_len = static_cast<uint32_t>(cur.end - cur.start);
        // the item's range cut to the query's causal window (inside the item)
        const int jhi = kVar ? min(cur.end, p + 1) : cur.end;
        const int jlo = (kVar && a.window > 0) ? max(cur.start, p - a.window + 1) : cur.start;
        vis_lo = jlo;
        vis_len = qlive && jhi > jlo ? static_cast<uint32_t>(jhi - jlo) : 0u;
      }
      m_run = kInitMax;
      l_run = 0.0f;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) oacc[dt] = mfma_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      // The next iteration's rows are always requested (past the item's end
      // the next item's, or a masked stand-in), so neither register set is
      // written conditionally: a conditional load made the compiler copy
      // whole register sets around the loop.  The late fetch acts at rounds
      // every wavefront reaches with real iterations, before any padding.
      int it = group_u;
      int rd = 0;
      while (it < num_iters) {
        late_fetch(rd);
        load_step(rb, it + kGroups, false);
        compute(ra, 0);
        it += kGroups;
        ++rd;
        late_fetch(rd);
        load_step(ra, it + kGroups, true);
        compute(rb, 1);                             // past the end: the masked stand-in
        it += kGroups;
        ++rd;
      }
    }
    // a wavefront without an iteration of this item requests its first rows
    // of the next one now
    if (group_u >= num_iters && nxt.valid && nxt.num_blk > 0) load_step(ra, num_iters, true);
    __syncthreads();                                 // every wavefront done with its V tile

    if (cur.num_blk > 0) {
      // this wavefront's partial: O^T column l16 rows 16dt+4gi+e; sum of weights
      // over the query's four lanes
      float lq = l_run;
      lq += __shfl_xor(lq, 16, 64);
      lq += __shfl_xor(lq, 32, 64);
      if (l16 < VG) {
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) sm.u.acc[wave][l16][16 * dt + 4 * gi + e] = oacc[dt][e];
        if (gi == 0) {
          sm.ml[wave][l16][0] = m_run;
          sm.ml[wave][l16][1] = lq;
        }
      }
    }
    // the next item's slice and queries (the queries' LDS is free again)
    if (nxt.valid) stage_store(nxt);
    __syncthreads();
    auto out_row = [&](int v) -> int64_t {
      if constexpr (kVar) {
        const int i = v / G;
        return i < cur.nq ? static_cast<int64_t>(cur.row0 + i) * a.num_q_heads + cur.g * G + (v - i * G) : -1;
      } else {
        return static_cast<int64_t>(cur.r) * a.num_q_heads + cur.g * G + v;
      }
    };
    if (cur.num_blk > 0) {
      const bool whole = a.split.single(cur.n - cur.lo);
      for (int e = tid; e < VG * D; e += kThreads) {
        const int h = e / D;
        const int d = e - h * D;
        const int64_t rh = out_row(h);
        if (rh < 0) continue;
        // the wavefronts holding column d: one per group (the wavefronts of
        // a group hold the same maximum and sum)
        const int dh = d / kDW;
        const int dd = d - dh * kDW;
        float mx = sm.ml[dh][h][0];
#pragma unroll
        for (int g = 1; g < kGroups; ++g) mx = fmaxf(mx, sm.ml[g * kSlices + dh][h][0]);
        float den = 0.0f, num = 0.0f;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          const int w = g * kSlices + dh;
          const float f = exp2f(sm.ml[w][h][0] - mx);
          den = fmaf(f, sm.ml[w][h][1], den);
          num = fmaf(f, sm.u.acc[w][h][dd], num);
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
      for (int e = tid; e < VG * D; e += kThreads) {
        const int h = e / D;
        const int64_t rh = out_row(h);
        if (rh >= 0) a.out[rh * D + (e - h * D)] = 0.0f;
      }
    }
    __syncthreads();                                 // sm reused by the next item
    cur = nxt;
    nxt = make_item(false, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, a.bs_shift);
  }


  if (tid == 0) {
    const uint32_t d = atomicAdd(done_ctr, 1u);
    if (d == gridDim.x - 1) {
      atomicExch(fetch_ctr, 0u);
      atomicExch(done_ctr, 0u);
    }
  }
}

}  // namespace yoco_attn
