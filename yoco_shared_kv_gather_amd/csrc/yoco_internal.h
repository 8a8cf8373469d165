// Internal helpers shared by the HIP sources of libyoco (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "yoco.h"

namespace yoco {

// ---- host side --------------------------------------------------------------

// Record a failure reason for yoco_last_error_message() and return `status`.
int32_t fail(int32_t status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clear any stale launch error on this thread (call right before a launch).
inline void clear_launch_error() { (void)hipGetLastError(); }

// Status of the launches enqueued since clear_launch_error().
int32_t launch_result(const char* what);

// Host copy of `count` int32 values at `src` (device or host memory), made on
// `stream` and waited for (validation mode only).  If the stream is being
// captured into a graph nothing may wait: `skip` is set and nothing copied.
int32_t fetch_indices(const int32_t* src, int64_t count, hipStream_t stream, std::vector<int32_t>& dst, bool& skip,
                      const char* who);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
inline int ilog2(int64_t v) { int s = 0; while ((int64_t(1) << s) < v) ++s; return s; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// ---- device side ------------------------------------------------------------

// bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// A 16-byte global load with the non-temporal hint (global_load ... nt), for
// rows a kernel streams through once, such as the K/V cache rows an attention
// layer reads: a plain streaming read reaches about 8% more bandwidth with it
// on gfx950.  Only for loads that take whole 128-byte lines per instruction:
// where one instruction reads half of each line and the next the other half,
// the hint costs a second fetch of the line.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}

// The same hint for 16 bytes of fp32 read or written once (a state that a
// kernel reads, updates and writes back).
__device__ __forceinline__ float4 load_stream_f4(const float* p) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const f32x4v w = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  return make_float4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ void store_stream_f4(float* p, const float4& v) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const f32x4v w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4v*>(p));
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two fp32 values -> packed bf16x2 (lo in bits 0-15), round to nearest even,
// with the hardware conversion (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
}

// fp32 -> FP8 E4M3 (finite-only variant: bias 7, no infinities, 0x7F/0xFF
// NaN, largest finite 448), rounded to nearest with ties to the even code.
// Magnitudes above 448 saturate to 448; NaN gives 0x7F.  Integer steps from
// the format definition, so the result does not depend on a conversion
// instruction's rounding or overflow mode.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                       // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;               // >= 448: saturate
  if (a < 0x3c800000u) {                                   // below 2^-6: subnormal codes m * 2^-9
    const float t = __uint_as_float(a) * 512.0f;           // exact scaling
    return sign | static_cast<uint32_t>(__builtin_rintf(t));   // 0..8 (8 is the smallest normal)
  }
  // normal: keep 3 of the 23 mantissa bits, ties to even, then rebias 127 -> 7
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  const uint32_t code = (r >> 20) - (120u << 3);
  return sign | (code < 0x7eu ? code : 0x7eu);
}

// E4M3 code of the fp32 quotient RN(y / s), given r = RN(1 / s) for finite
// s > 0 (pass r = 0 where the caller overrides the code anyway).  Mostly
// without a division: q' = RN(y r) is within 2^-23 |y/s| of y/s, so RN(y/s)
// lies between RN(q'(1 - 2^-21)) and RN(q'(1 + 2^-21)); the hardware
// encoder (round to nearest even; on every finite input below 464 in
// magnitude it gives f32_to_e4m3_rne's code) takes both, and since the
// encoding is monotone in the magnitude, a common code is the quotient's.
// Where they differ (a rounding midpoint within reach, a few values in a
// million) or r is infinite, the quotient is divided out.
__device__ __forceinline__ uint32_t e4m3_of_quotient(float y, float s, float r) {
  const float q = y * r;
  const uint32_t pk = static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(q * (1.0f - 0x1p-21f), q * (1.0f + 0x1p-21f), 0, false));
  const uint32_t c = pk & 0xffu;
  if (c == ((pk >> 8) & 0xffu) && r < __builtin_inff()) return c;
  return f32_to_e4m3_rne(y / s);
}

}  // namespace yoco
