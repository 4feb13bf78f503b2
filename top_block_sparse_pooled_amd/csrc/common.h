// Shared definitions of the gfx950 kernels: vector types, bf16 conversions, launch checks.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "fvattn.h"

namespace fv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef double d4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bit pattern, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f2bf(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

template <typename T> struct DT;
template <> struct DT<uint16_t> { static constexpr int per16 = 8; };  // bf16 stored as u16
template <> struct DT<float> { static constexpr int per16 = 4; };

// Unpack one 16-byte chunk into float values.
__device__ __forceinline__ void unpack16(const u32x4 &c, float *out, uint16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf16_lo(c[i]);
    out[2 * i + 1] = bf16_hi(c[i]);
  }
}
__device__ __forceinline__ void unpack16(const u32x4 &c, float *out, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(c[i]);
}

__host__ __device__ constexpr inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Control block of an attention plan: int32[64] at the start of the attention workspace.
namespace ctl {
constexpr int kTicket = 0;      // next unit of the single queue
constexpr int kExit = 1;        // workgroups that have left (the last one restores the tickets)
constexpr int kPerXcd = 2;      // 1: per-XCD queues with stealing
constexpr int kXcdTicket = 8;   // [8]: next unit of XCD x's queue
constexpr int kXcdStart = 16;   // [9]: first unit of XCD x's queue; [16 + 8] = units
constexpr int kSig = 32;        // plan signature: units, G, dtype, nqb, bh, nkb, n, magic
constexpr int kSigLen = 8;
constexpr int kStatus = 40;     // FVATTN_STATUS_* bits set by the attention kernels
constexpr int kMagic = 0x46565032;
constexpr int kWords = 64;
}  // namespace ctl

// Smallest shift with (width - 1) >> shift < 256: the 8-bit radix digit of a key in a range of
// `width` keys (radix selects over float64 bit patterns).
__device__ __forceinline__ int digit_shift(unsigned long long width) {
  const unsigned long long wm1 = width - 1ull;
  return wm1 < 256ull ? 0 : 64 - __clzll((long long)wm1) - 8;
}

// s_waitcnt on the vector memory counter only (expcnt and lgkmcnt fields at their maxima).
template <int NV>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(NV >= 0 && NV < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((NV & 15) | ((NV >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Compute units of the current device (cached per device); 0 on success.
inline int device_cus(int *cus) {
  // per-device cache; concurrent callers may both query and store the same value
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return 0;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return 0;
}

}  // namespace fv

// Returns FVATTN_ERR_HIP from the enclosing function if the last launch failed.
#define FV_CHECK_LAUNCH()                                   \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return FVATTN_ERR_HIP; \
  } while (0)
