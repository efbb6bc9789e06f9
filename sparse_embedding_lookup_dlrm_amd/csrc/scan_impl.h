// Device-wide exclusive prefix sums over int32 sequences (three passes: chunk
// totals, a one-workgroup scan of the totals, chunk fill). The input is a
// functor so the backward can scan flags it never materialises.
#pragma once

#include "common.h"

namespace dlrm {

constexpr int kScanThreads = 256;
constexpr int kScanPerThread = 16;
constexpr int kScanChunk = kScanThreads * kScanPerThread;  // 4096 items per workgroup

// Exclusive scan of one value per thread across the workgroup; *total gets the sum.
__device__ __forceinline__ long long block_exclusive_scan(long long v, long long* total, long long* lds) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  constexpr int nw = kScanThreads / kWave;
  long long x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) lds[wave] = x;
  __syncthreads();
  long long base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < nw; ++w) {
    const long long s = lds[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

struct ArrayIn {
  const int32_t* p;
  __device__ __forceinline__ long long operator()(long long i) const { return p[i]; }
};

// Chunk totals -> partial[c].
template <class In>
__global__ __launch_bounds__(kScanThreads) void scan_chunk_totals(In in, long long n, long long* partial) {
  __shared__ long long lds[kScanThreads / kWave];
  const long long c0 = static_cast<long long>(blockIdx.x) * kScanChunk + threadIdx.x * kScanPerThread;
  long long s = 0;
#pragma unroll
  for (int k = 0; k < kScanPerThread; ++k)
    if (c0 + k < n) s += in(c0 + k);
  long long tot;
  block_exclusive_scan(s, &tot, lds);
  if (threadIdx.x == 0) partial[blockIdx.x] = tot;
}

// partial[0..m) -> exclusive prefix, partial[m] = grand total. One workgroup.
static __global__ __launch_bounds__(kScanThreads) void scan_partials(long long* partial, long long m) {
  __shared__ long long lds[kScanThreads / kWave];
  long long carry = 0;
  for (long long base = 0; base < m; base += kScanChunk) {
    const long long c0 = base + threadIdx.x * kScanPerThread;
    long long v[kScanPerThread];
    long long s = 0;
#pragma unroll
    for (int k = 0; k < kScanPerThread; ++k) {
      v[k] = (c0 + k < m) ? partial[c0 + k] : 0;
      s += v[k];
    }
    long long tot;
    long long ex = block_exclusive_scan(s, &tot, lds) + carry;
#pragma unroll
    for (int k = 0; k < kScanPerThread; ++k) {
      if (c0 + k < m) partial[c0 + k] = ex;
      ex += v[k];
    }
    carry += tot;
  }
  if (threadIdx.x == 0) partial[m] = carry;
}

// out[i] = partial[chunk] + prefix inside the chunk; out[n] = total. Values are
// stored as int32; `overflow` is raised (status bit) when the total exceeds INT32_MAX.
template <class In>
__global__ __launch_bounds__(kScanThreads) void scan_chunk_fill(In in, long long n, const long long* partial,
                                                                int32_t* out, int32_t* status, int overflow_bit) {
  __shared__ long long lds[kScanThreads / kWave];
  const long long c0 = static_cast<long long>(blockIdx.x) * kScanChunk + threadIdx.x * kScanPerThread;
  long long v[kScanPerThread];
  long long s = 0;
#pragma unroll
  for (int k = 0; k < kScanPerThread; ++k) {
    v[k] = (c0 + k < n) ? in(c0 + k) : 0;
    s += v[k];
  }
  long long tot;
  long long ex = block_exclusive_scan(s, &tot, lds) + partial[blockIdx.x];
#pragma unroll
  for (int k = 0; k < kScanPerThread; ++k) {
    if (c0 + k < n) out[c0 + k] = static_cast<int32_t>(ex);
    ex += v[k];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const long long total = partial[gridDim.x];
    out[n] = static_cast<int32_t>(total);
    if (total > 0x7fffffffLL && overflow_bit) flag(status, overflow_bit);
  }
}

inline long long scan_chunks(long long n) { return (n + kScanChunk - 1) / kScanChunk; }

// Exclusive scan of in[0..n) into out[0..n], out[n] = total. partial needs
// scan_chunks(n) + 1 int64 entries of device memory. n >= 1.
template <class In>
hipError_t device_exclusive_scan(In in, long long n, int32_t* out, long long* partial, int32_t* status,
                                 int overflow_bit, hipStream_t st) {
  const long long m = scan_chunks(n);
  hipLaunchKernelGGL((scan_chunk_totals<In>), dim3(static_cast<unsigned>(m)), dim3(kScanThreads), 0, st, in, n,
                     partial);
  hipLaunchKernelGGL(scan_partials, dim3(1), dim3(kScanThreads), 0, st, partial, m);
  hipLaunchKernelGGL((scan_chunk_fill<In>), dim3(static_cast<unsigned>(m)), dim3(kScanThreads), 0, st, in, n,
                     partial, out, status, overflow_bit);
  return hipGetLastError();
}

}  // namespace dlrm
