// Bag lengths -> CSR offsets (exclusive prefix sum) without a workspace: the
// total of chunk c is parked in offsets[end of chunk c], which is exactly the
// slot that ends up holding the inclusive prefix at that chunk boundary.
#include "scan_impl.h"

namespace dlrm {

__device__ __forceinline__ long long clamp_len(int32_t v, bool& bad) {
  if (v < 0) { bad = true; return 0; }
  return v;
}

__global__ __launch_bounds__(kScanThreads) void l2o_totals(long long n, const int32_t* __restrict__ len,
                                                           int32_t* __restrict__ off, int32_t* status) {
  __shared__ long long lds[kScanThreads / kWave];
  const long long c0 = static_cast<long long>(blockIdx.x) * kScanChunk + threadIdx.x * kScanPerThread;
  long long s = 0;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kScanPerThread; ++k)
    if (c0 + k < n) s += clamp_len(len[c0 + k], bad);
  if (bad) flag(status, DLRM_STATUS_BAD_OFFSETS);
  long long tot;
  block_exclusive_scan(s, &tot, lds);
  if (threadIdx.x == 0) {
    long long end = static_cast<long long>(blockIdx.x + 1) * kScanChunk;
    if (end > n) end = n;
    if (tot > 0x7fffffffLL) {
      tot = 0x7fffffffLL;
      flag(status, DLRM_STATUS_BAD_OFFSETS);
    }
    off[end] = static_cast<int32_t>(tot);
  }
}

__global__ __launch_bounds__(kScanThreads) void l2o_scan(long long n, long long m, int32_t* __restrict__ off,
                                                         int32_t* status) {
  __shared__ long long lds[kScanThreads / kWave];
  long long carry = 0;
  bool over = false;
  for (long long base = 0; base < m; base += kScanChunk) {
    const long long c0 = base + threadIdx.x * kScanPerThread;
    long long v[kScanPerThread];
    long long s = 0;
#pragma unroll
    for (int k = 0; k < kScanPerThread; ++k) {
      const long long c = c0 + k;
      long long e = (c + 1) * kScanChunk;
      if (e > n) e = n;
      v[k] = (c < m) ? off[e] : 0;
      s += v[k];
    }
    long long tot;
    long long inc = block_exclusive_scan(s, &tot, lds) + carry;
#pragma unroll
    for (int k = 0; k < kScanPerThread; ++k) {
      const long long c = c0 + k;
      inc += v[k];
      if (c < m) {
        long long e = (c + 1) * kScanChunk;
        if (e > n) e = n;
        if (inc > 0x7fffffffLL) over = true;
        off[e] = static_cast<int32_t>(inc > 0x7fffffffLL ? 0x7fffffffLL : inc);
      }
    }
    carry += tot;
  }
  if (over) flag(status, DLRM_STATUS_BAD_OFFSETS);
  if (threadIdx.x == 0) off[0] = 0;
}

__global__ __launch_bounds__(kScanThreads) void l2o_fill(long long n, const int32_t* __restrict__ len,
                                                         int32_t* __restrict__ off) {
  __shared__ long long lds[kScanThreads / kWave];
  const long long chunk0 = static_cast<long long>(blockIdx.x) * kScanChunk;
  long long chunk_end = chunk0 + kScanChunk;
  if (chunk_end > n) chunk_end = n;
  const long long c0 = chunk0 + threadIdx.x * kScanPerThread;
  long long v[kScanPerThread];
  long long s = 0;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kScanPerThread; ++k) {
    v[k] = (c0 + k < n) ? clamp_len(len[c0 + k], bad) : 0;
    s += v[k];
  }
  long long tot;
  const long long base = blockIdx.x == 0 ? 0 : static_cast<long long>(off[chunk0]);
  long long inc = block_exclusive_scan(s, &tot, lds) + base;
#pragma unroll
  for (int k = 0; k < kScanPerThread; ++k) {
    const long long i = c0 + k;
    inc += v[k];
    // the last item of the chunk ends at off[chunk_end], already written by l2o_scan
    if (i < chunk_end - 1) off[i + 1] = static_cast<int32_t>(inc > 0x7fffffffLL ? 0x7fffffffLL : inc);
  }
}

// One workgroup writes offsets[0] = 0 for an empty batch.
__global__ void l2o_empty(int32_t* off) {
  if (threadIdx.x == 0) off[0] = 0;
}

hipError_t launch_lengths_to_offsets(int64_t n, const int32_t* lengths, int32_t* offsets, int32_t* status,
                                     hipStream_t st) {
  if (n == 0) {
    hipLaunchKernelGGL(l2o_empty, dim3(1), dim3(64), 0, st, offsets);
    return hipGetLastError();
  }
  const long long m = scan_chunks(n);
  hipLaunchKernelGGL(l2o_totals, dim3(static_cast<unsigned>(m)), dim3(kScanThreads), 0, st, (long long)n, lengths,
                     offsets, status);
  hipLaunchKernelGGL(l2o_scan, dim3(1), dim3(kScanThreads), 0, st, (long long)n, m, offsets, status);
  hipLaunchKernelGGL(l2o_fill, dim3(static_cast<unsigned>(m)), dim3(kScanThreads), 0, st, (long long)n, lengths,
                     offsets);
  return hipGetLastError();
}

}  // namespace dlrm
