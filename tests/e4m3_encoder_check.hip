// Check, on the GPU it runs on, the two facts the FP8 quantizers' fast path
// stands on:
//  1. the hardware E4M3 encoder (v_cvt_pk_fp8_f32, round to nearest even)
//     gives yoco::f32_to_e4m3_rne's code for every finite fp32 input below
//     464 in magnitude, both signs (all 2^31 + ... such bit patterns);
//  2. yoco::e4m3_of_quotient(y, s, 1/s) equals f32_to_e4m3_rne(y / s) on
//     random rows (a row max m, s = m / 448, y = m t with |t| <= 1 spread
//     over 40 binades, and y = +-m itself), 2^31 cases per seed.
// Prints one line per check; exit status 0 when both hold.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "yoco_internal.h"

namespace {

constexpr uint32_t kLimit = 0x43E80000u;    // bit pattern of 464.0f
constexpr int kThreads = 256;
constexpr int kBlocks = 8192;
constexpr int kTotal = kThreads * kBlocks;  // one result slot per thread
constexpr int kPerThread = 1024;            // quotient cases per thread and seed

__global__ __launch_bounds__(kThreads) void encoder_check(uint32_t* bad, uint32_t* first) {
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t per = (kLimit + kTotal - 1) / kTotal;
  const uint32_t lo = static_cast<uint32_t>(gid) * per;
  const uint32_t hi = lo + per < kLimit ? lo + per : kLimit;
  uint32_t n = 0, f = 0xFFFFFFFFu;
  for (uint32_t a = lo; a < hi; ++a) {
    for (uint32_t sign = 0; sign < 2; ++sign) {
      const uint32_t u = a | (sign << 31);
      const float x = __uint_as_float(u);
      const uint32_t hw = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false)) & 0xFFFFu;
      const uint32_t sw = yoco::f32_to_e4m3_rne(x);
      if ((hw & 0xFFu) != sw || (hw >> 8) != sw) {
        ++n;
        if (f == 0xFFFFFFFFu) f = u;
      }
    }
  }
  bad[gid] = n;
  first[gid] = f;
}

__device__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(kThreads) void quotient_check(uint32_t* bad, uint32_t seed) {
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  uint32_t n = 0;
  for (int it = 0; it < kPerThread; ++it) {
    const uint32_t h1 = mix32(seed ^ mix32(static_cast<uint32_t>(gid) * kPerThread + it));
    const uint32_t h2 = mix32(h1 + 0x9e3779b9u);
    const uint32_t h3 = mix32(h2 + 0x85ebca6bu);
    const float m = ldexpf(1.0f + (h1 & 0xFFFFFFu) * 0x1p-24f, static_cast<int>(h2 % 141u) - 100);
    float t = (h3 & 0xFFFFFFu) * 0x1p-24f * ((h3 >> 31) ? -1.0f : 1.0f);
    t = ldexpf(t, -static_cast<int>((h2 >> 16) % 41u));
    if ((h1 >> 28) == 0) t = (h3 >> 31) ? -1.0f : 1.0f;
    const float y = m * t;
    const float s = m / 448.0f;
    const uint32_t exact = yoco::f32_to_e4m3_rne(y / s);
    const uint32_t fast = yoco::e4m3_of_quotient(y, s, 1.0f / s);
    n += exact != fast;
  }
  bad[gid] = n;
}

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) std::printf("%s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

}  // namespace

int main() {
  uint32_t* bad = nullptr;
  uint32_t* first = nullptr;
  if (!ok(hipMalloc(&bad, kTotal * sizeof(uint32_t)), "hipMalloc") ||
      !ok(hipMalloc(&first, kTotal * sizeof(uint32_t)), "hipMalloc"))
    return 2;
  std::vector<uint32_t> b(kTotal), f(kTotal);
  hipLaunchKernelGGL(encoder_check, dim3(kBlocks), dim3(kThreads), 0, 0, bad, first);
  if (!ok(hipGetLastError(), "encoder_check launch") || !ok(hipDeviceSynchronize(), "encoder_check") ||
      !ok(hipMemcpy(b.data(), bad, kTotal * sizeof(uint32_t), hipMemcpyDeviceToHost), "copy") ||
      !ok(hipMemcpy(f.data(), first, kTotal * sizeof(uint32_t), hipMemcpyDeviceToHost), "copy"))
    return 2;
  uint64_t enc_bad = 0;
  int shown = 0;
  for (int i = 0; i < kTotal; ++i) {
    enc_bad += b[i];
    if (b[i] != 0 && shown < 8) {
      std::printf("encoder differs at input 0x%08x\n", f[i]);
      ++shown;
    }
  }
  std::printf("encoder: %llu of %llu inputs differ\n", static_cast<unsigned long long>(enc_bad),
              2ull * kLimit);
  uint64_t quo_bad = 0;
  constexpr uint32_t kSeeds = 16;
  for (uint32_t seed = 1; seed <= kSeeds; ++seed) {
    hipLaunchKernelGGL(quotient_check, dim3(kBlocks), dim3(kThreads), 0, 0, bad, seed);
    if (!ok(hipGetLastError(), "quotient_check launch") || !ok(hipDeviceSynchronize(), "quotient_check") ||
        !ok(hipMemcpy(b.data(), bad, kTotal * sizeof(uint32_t), hipMemcpyDeviceToHost), "copy"))
      return 2;
    for (int i = 0; i < kTotal; ++i) quo_bad += b[i];
  }
  std::printf("quotient: %llu of %llu cases differ\n", static_cast<unsigned long long>(quo_bad),
              static_cast<unsigned long long>(kSeeds) * kTotal * kPerThread);
  ok(hipFree(bad), "hipFree");
  ok(hipFree(first), "hipFree");
  return enc_bad == 0 && quo_bad == 0 ? 0 : 1;
}
