// Internal device/host helpers shared by the HIP kernels of libdlrm_embbag.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "dlrm_embbag.h"
#include "launch.h"

namespace dlrm {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// storage formats
// ---------------------------------------------------------------------------
template <int DT>
struct Storage;
template <>
struct Storage<DLRM_F32> {
  static constexpr int bytes = 4;
  static constexpr int per16 = 4;  // elements per 16-byte load
};
template <>
struct Storage<DLRM_F16> {
  static constexpr int bytes = 2;
  static constexpr int per16 = 8;
};
template <>
struct Storage<DLRM_BF16> {
  static constexpr int bytes = 2;
  static constexpr int per16 = 8;
};
template <>
struct Storage<DLRM_Q4> {
  static constexpr int bytes = 1;   // a code byte (two columns)
  static constexpr int per16 = 32;
};
template <>
struct Storage<DLRM_Q8T> {
  static constexpr int bytes = 1;
  static constexpr int per16 = 16;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16)));
}

// acc[0..per16) += the 16 bytes in v, decoded from the storage type (exact widening to fp32).
template <int DT>
__device__ __forceinline__ void accumulate16(float* acc, const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (DT == DLRM_F32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += __uint_as_float(w[k]);
  } else if constexpr (DT == DLRM_BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += bf16_lo(w[k]);
      acc[2 * k + 1] += bf16_hi(w[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += f16_lo(w[k]);
      acc[2 * k + 1] += f16_hi(w[k]);
    }
  }
}

// fp32 -> storage, round to nearest even (finite inputs; NaN stays NaN).
template <int DT>
__device__ __forceinline__ uint16_t to_half_bits(float x);
template <>
__device__ __forceinline__ uint16_t to_half_bits<DLRM_BF16>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
template <>
__device__ __forceinline__ uint16_t to_half_bits<DLRM_F16>(float x) {
  return __half_as_ushort(__float2half_rn(x));
}

// 16-byte streaming load: table rows are read once per lookup, so they bypass
// the cache-retention policy (non-temporal) and leave L2/MALL to the indices.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const uint32_t* q = static_cast<const uint32_t*>(p);
  uint4 v;
  v.x = __builtin_nontemporal_load(q + 0);
  v.y = __builtin_nontemporal_load(q + 1);
  v.z = __builtin_nontemporal_load(q + 2);
  v.w = __builtin_nontemporal_load(q + 3);
  return v;
}

__device__ __forceinline__ void store_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ void flag(int32_t* status, int bits) {
  if (status) atomicOr(status, bits);
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical blocks so that neighbouring samples (which share
// cache lines of offsets/indices) meet in the same L2.
__device__ __forceinline__ int xcd_block(int bid, int n) {
  const int xcd = bid & 7, k = bid >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + k;
}

__device__ __forceinline__ int shfl_i(int v, int src) { return __shfl(v, src, kWave); }
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

}  // namespace dlrm

