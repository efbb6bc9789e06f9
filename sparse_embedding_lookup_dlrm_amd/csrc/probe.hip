// Measurement kernel: the bare random-row gather of a batch, with the same
// one-row-per-wave-wide-load access as the row-streaming forward and nothing
// else (no bags, no pooling order, no interaction, no output rows). Its time is
// the ceiling the fused forward is compared against.
#include "common.h"
#include "dlrm_probe.h"

namespace dlrm {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeGrid = 4096;  // workgroups (16 per CU)

struct ProbeArgs {
  const void* ptr[DLRM_MAX_TABLES];
  int32_t rows[DLRM_MAX_TABLES];
  int64_t start[DLRM_MAX_TABLES + 1];  // first CSR position of each table
  int T;
  const int32_t* indices;
  int64_t nnz;
};

template <int LB>
struct Chunk;
template <>
struct Chunk<2> {
  using type = uint32_t;
  __device__ static type load(uint64_t p) {
    return __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) uint16_t*>(p));
  }
  __device__ static float sum(type v) { return __uint_as_float(v << 16); }
};
template <>
struct Chunk<4> {
  using type = uint32_t;
  __device__ static type load(uint64_t p) {
    return __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(p));
  }
  __device__ static float sum(type v) { return __uint_as_float(v); }
};
template <>
struct Chunk<8> {
  using type = uint2;
  __device__ static type load(uint64_t p) {
    const auto q = reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(p);
    return make_uint2(__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1));
  }
  __device__ static float sum(type v) { return __uint_as_float(v.x) + __uint_as_float(v.y); }
};
template <>
struct Chunk<16> {
  using type = uint4;
  __device__ static type load(uint64_t p) {
    const auto q = reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(p);
    return make_uint4(__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                      __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3));
  }
  __device__ static float sum(type v) {
    return (__uint_as_float(v.x) + __uint_as_float(v.y)) + (__uint_as_float(v.z) + __uint_as_float(v.w));
  }
};

__device__ __forceinline__ uint64_t bcast(uint64_t a, int j) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(a & 0xffffffffu), j));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(a >> 32), j));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Largest t in [0, T) with start[t] <= p (start non-decreasing, start[0] = 0).
__device__ __forceinline__ int table_of(const int* start, int T, int p) {
  int lo = 0;
#pragma unroll
  for (int step = 64; step > 0; step >>= 1) {
    const int c = lo + step;
    if (c < T && start[c] <= p) lo = c;
  }
  return lo;
}

// Each wave streams a contiguous range of positions, 64 at a time: lane l
// works out the address of position q + l (table by a search over the table
// boundaries in LDS, index prefetched one chunk ahead), then the wave reads
// the rows one wave-wide load each in two windows of 32, the next window always
// issued before the previous one is summed, so 32 to 64 rows stay in flight.
template <int LB>
__global__ __launch_bounds__(kProbeThreads) void probe_gather_kernel(ProbeArgs a, float* __restrict__ sink) {
  using C = Chunk<LB>;
  constexpr int RB = LB * kWave;
  constexpr int HALF = kWave / 2;
  __shared__ int start[DLRM_MAX_TABLES + 1];
  __shared__ uint64_t base[DLRM_MAX_TABLES];
  __shared__ int rows[DLRM_MAX_TABLES];
  for (int t = threadIdx.x; t <= a.T; t += kProbeThreads) start[t] = static_cast<int>(a.start[t]);
  for (int t = threadIdx.x; t < a.T; t += kProbeThreads) {
    base[t] = reinterpret_cast<uint64_t>(a.ptr[t]);
    rows[t] = a.rows[t];
  }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * (kProbeThreads / kWave) + (threadIdx.x >> 6);
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (kProbeThreads / kWave);
  const int64_t nchunks = (a.nnz + kWave - 1) / kWave;
  const int64_t c0 = nchunks * gw / nw, c1 = nchunks * (gw + 1) / nw;
  if (c0 >= c1) return;
  const int n = static_cast<int>(a.nnz);
  const uint64_t lane_off = static_cast<uint64_t>(lane) * LB;
  auto index_of = [&](int64_t c) -> int {  // in bounds for any chunk of the range
    const int64_t p = c * kWave + lane;
    return a.indices[p < n ? p : n - 1];
  };
  auto address = [&](int64_t c, int r) -> uint64_t {
    const int p = static_cast<int>(c * kWave + lane);
    const int t = table_of(start, a.T, p < n ? p : n - 1);
    const bool ok = p < n && r >= 0 && r < rows[t];
    return base[ok ? t : 0] + (ok ? static_cast<uint64_t>(r) * RB : 0);
  };
  float acc = 0.f;
  typename C::type va[HALF], vb[HALF];
  uint64_t cur = address(c0, index_of(c0));
  int nidx = index_of(c0 + 1 < c1 ? c0 + 1 : c0);
#pragma unroll
  for (int j = 0; j < HALF; ++j) va[j] = C::load(bcast(cur, j) + lane_off);
  for (int64_t c = c0; c < c1; ++c) {
#pragma unroll
    for (int j = 0; j < HALF; ++j) vb[j] = C::load(bcast(cur, HALF + j) + lane_off);
#pragma unroll
    for (int j = 0; j < HALF; ++j) acc += C::sum(va[j]);
    if (c + 1 < c1) {  // wave-uniform
      cur = address(c + 1, nidx);
      nidx = index_of(c + 2 < c1 ? c + 2 : c + 1);
#pragma unroll
      for (int j = 0; j < HALF; ++j) va[j] = C::load(bcast(cur, j) + lane_off);
    }
#pragma unroll
    for (int j = 0; j < HALF; ++j) acc += C::sum(vb[j]);
  }
  sink[static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

}  // namespace dlrm

extern "C" int dlrm_probe_row_gather(int32_t T, int32_t D, int32_t dtype, const void* const* tables,
                                     const int64_t* rows, const int64_t* table_start, const int32_t* indices,
                                     int64_t nnz, float* sink, void* stream) {
  using namespace dlrm;
  if (T < 1 || T > DLRM_MAX_TABLES || D < 1 || nnz < 1 || !tables || !rows || !table_start || !indices || !sink)
    return DLRM_E_INVAL;
  const int s = dtype == DLRM_F32 ? 4 : (dtype == DLRM_F16 || dtype == DLRM_BF16) ? 2 : 0;
  const long rb = static_cast<long>(D) * s;
  if (s == 0 || rb < 128 || rb > 1024 || (rb & (rb - 1)) != 0) return DLRM_E_UNSUPPORTED;
  ProbeArgs a{};
  a.T = T;
  a.indices = indices;
  a.nnz = nnz;
  for (int t = 0; t < T; ++t) {
    if (!tables[t] || rows[t] < 1 || rows[t] > 0x7fffffffLL) return DLRM_E_INVAL;
    a.ptr[t] = tables[t];
    a.rows[t] = static_cast<int32_t>(rows[t]);
  }
  for (int t = 0; t <= T; ++t) a.start[t] = table_start[t];
  if (nnz >= 0x7fffffffLL) return DLRM_E_INVAL;
  // a few thousand workgroups, each wave streaming a contiguous range of positions
  const int64_t chunks = (nnz + kWave - 1) / kWave;
  const int64_t want = (chunks + (kProbeThreads / kWave) - 1) / (kProbeThreads / kWave);
  const int grid = static_cast<int>(want < kProbeGrid ? want : kProbeGrid);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (rb / 64) {
    case 2: hipLaunchKernelGGL(probe_gather_kernel<2>, dim3(grid), dim3(kProbeThreads), 0, st, a, sink); break;
    case 4: hipLaunchKernelGGL(probe_gather_kernel<4>, dim3(grid), dim3(kProbeThreads), 0, st, a, sink); break;
    case 8: hipLaunchKernelGGL(probe_gather_kernel<8>, dim3(grid), dim3(kProbeThreads), 0, st, a, sink); break;
    default: hipLaunchKernelGGL(probe_gather_kernel<16>, dim3(grid), dim3(kProbeThreads), 0, st, a, sink); break;
  }
  return hipGetLastError() == hipSuccess ? DLRM_OK : DLRM_E_HIP;
}
