// Embedding-bag forward (gather + sum-pool) and the pairwise dot-product
// interaction, for gfx950.
//
// What is computed ("DLRM" note, sections 2 and 3): for every sample b and
// table t, pooled[b][t] = sum of the table-t rows named by bag (t, b); then
// Z[b] = [e0[b]; pooled[b][0..T)] and out[b] = [e0[b] | Z[b][i].Z[b][j], i > j].
//
// Gather: LPR lanes read one table row with 16-byte loads (LPR = row bytes/16),
// so a wave covers R = 64/LPR rows per load instruction; each wave keeps U
// such loads in flight per bag and works on two bags at once. Indices come in
// one coalesced 64-wide load per chunk and are handed to the row lanes by
// cross-lane permutes. Rows are summed in fp32 registers in a fixed order
// (row slot order, then a butterfly across the R row groups), so results are
// deterministic.
//
// Fused path: the pooled vectors of a workgroup's samples go straight into an
// LDS tile Z[s][F][D] (fp32), e0 fills row 0, and the strict-lower dots are
// computed from LDS with 4x4 register blocks. Nothing but [e0 | dots] reaches
// HBM.
#include "common.h"

namespace dlrm {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kBagsPerWave = 2;

template <int DT, int LPR>
struct GatherShape {
  static constexpr int R = kWave / LPR;             // rows per wave-wide load
  static constexpr int EL = Storage<DT>::per16;     // elements per lane per load
  static constexpr int U = (R * 8 <= kWave) ? 8 : kWave / R;  // loads in flight per bag
  static constexpr int CH = R * U;                  // rows per chunk (<= 64)
  static_assert(CH <= kWave, "one index load per chunk");
};

// Sum-pools NB bags of one wave. t/begin/n are wave-uniform. On return the
// lanes with lane < LPR hold elements [lane*EL, lane*EL+EL) of each bag's sum.
template <int DT, int LPR, int NB>
__device__ __forceinline__ void gather_bags(const TableArgs& tabs, const int32_t* __restrict__ indices,
                                            const int (&t)[NB], const int (&begin)[NB], const int (&n)[NB],
                                            float (&acc)[NB][GatherShape<DT, LPR>::EL], int32_t* status) {
  using G = GatherShape<DT, LPR>;
  constexpr int ROWB = LPR * 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane / LPR, sub = lane % LPR;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < G::EL; ++e) acc[b][e] = 0.f;

  int nmax = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) nmax = n[b] > nmax ? n[b] : nmax;

  for (int c = 0; c < nmax; c += G::CH) {
    int my[NB];
    bool bad = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int pos = c + lane;
      my[b] = -1;
      if (lane < G::CH && pos < n[b]) {
        const int r = indices[begin[b] + pos];
        if (r >= 0 && r < tabs.rows[t[b]]) my[b] = r;
        else bad = true;
      }
    }
    if (bad) flag(status, DLRM_STATUS_BAD_INDEX);
    uint4 v[NB][G::U];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const char* base = static_cast<const char*>(tabs.ptr[t[b]]) + sub * 16;
#pragma unroll
      for (int u = 0; u < G::U; ++u) {
        const int r = shfl_i(my[b], u * G::R + grp);
        if (r >= 0) v[b][u] = load16_stream(base + static_cast<size_t>(r) * ROWB);
        else v[b][u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int u = 0; u < G::U; ++u) accumulate16<DT>(acc[b], v[b][u]);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < G::EL; ++e)
#pragma unroll
      for (int m = LPR; m < kWave; m <<= 1) acc[b][e] += shfl_xor_f(acc[b][e], m);
}

// Clamp a bag's CSR range into [0, nnz] and report anything that is not a valid CSR.
__device__ __forceinline__ void check_range(int t, int b, int T, int B, int64_t nnz, int& begin, int& end,
                                            int32_t* status) {
  bool bad = false;
  if (t == 0 && b == 0 && begin != 0) bad = true;
  if (t == T - 1 && b == B - 1 && static_cast<int64_t>(end) != nnz) bad = true;
  if (begin < 0) { begin = 0; bad = true; }
  if (static_cast<int64_t>(begin) > nnz) { begin = static_cast<int>(nnz); bad = true; }
  if (static_cast<int64_t>(end) > nnz) { end = static_cast<int>(nnz); bad = true; }
  if (end < begin) { end = begin; bad = true; }
  if (bad && (threadIdx.x & (kWave - 1)) == 0) flag(status, DLRM_STATUS_BAD_OFFSETS);
}

// ---------------------------------------------------------------------------
// pooled-only forward: one wave per two bags, output pooled[b][t][:]
// ---------------------------------------------------------------------------
template <int DT, int LPR>
__global__ __launch_bounds__(kThreads) void pool_kernel(FwdArgs a) {
  using G = GatherShape<DT, LPR>;
  constexpr int NB = kBagsPerWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * kWavesPerBlock + wave;
  const int nw = gridDim.x * kWavesPerBlock;
  const int nbags = a.T * a.B;
  const int lane = threadIdx.x & (kWave - 1);
  for (int j0 = gw * NB; j0 < nbags; j0 += nw * NB) {
    int t[NB], begin[NB], n[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = j0 + b;
      t[b] = 0; begin[b] = 0; n[b] = 0;
      if (j < nbags) {
        const int smp = j / a.T, tt = j - smp * a.T;
        int s0 = a.offsets[tt * a.B + smp], s1 = a.offsets[tt * a.B + smp + 1];
        check_range(tt, smp, a.T, a.B, a.nnz, s0, s1, a.status);
        t[b] = tt; begin[b] = __builtin_amdgcn_readfirstlane(s0);
        n[b] = __builtin_amdgcn_readfirstlane(s1 - s0);
      }
    }
    float acc[NB][G::EL];
    gather_bags<DT, LPR, NB>(a.tabs, a.indices, t, begin, n, acc, a.status);
    if (lane < LPR) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int j = j0 + b;
        if (j < nbags) {
          float* o = a.out_pooled + static_cast<size_t>(j) * a.D + lane * G::EL;
#pragma unroll
          for (int e = 0; e < G::EL; e += 4)
            *reinterpret_cast<float4*>(o + e) = make_float4(acc[b][e], acc[b][e + 1], acc[b][e + 2], acc[b][e + 3]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// interaction from an LDS tile: 4x4 register blocks of the strict lower triangle
// ---------------------------------------------------------------------------
__device__ __forceinline__ void block_pair(int w, int& bi, int& bj) {
  int i = static_cast<int>((sqrtf(8.f * w + 1.f) - 1.f) * 0.5f);
  while (i * (i + 1) / 2 > w) --i;
  while ((i + 1) * (i + 2) / 2 <= w) ++i;
  bi = i;
  bj = w - i * (i + 1) / 2;
}

// Z: [Fpad][LD] fp32 in LDS (rows >= F may hold anything); dots of block (bi, bj)
// for i in 4bi..4bi+3, j in 4bj..4bj+3 with j < i < F go to out[i(i-1)/2 + j].
__device__ __forceinline__ void dots_block(const float* Z, int F, int D, int LD, int bi, int bj,
                                           float* __restrict__ out) {
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[r][q] = 0.f;
  const float* zi = Z + (4 * bi) * LD;
  const float* zj = Z + (4 * bj) * LD;
  for (int d = 0; d < D; d += 4) {
    float4 x[4], y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = *reinterpret_cast<const float4*>(zi + r * LD + d);
      y[r] = *reinterpret_cast<const float4*>(zj + r * LD + d);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float s = acc[r][q];
        s = fmaf(x[r].x, y[q].x, s);
        s = fmaf(x[r].y, y[q].y, s);
        s = fmaf(x[r].z, y[q].z, s);
        s = fmaf(x[r].w, y[q].w, s);
        acc[r][q] = s;
      }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * bi + r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = 4 * bj + q;
      if (i < F && j < i) store_stream(out + (i * (i - 1) / 2 + j), acc[r][q]);
    }
  }
}

struct Tile {
  int S;      // samples per workgroup
  int F;      // T + 1
  int Fpad;   // F rounded up to 4
  int LD;     // LDS row stride (floats)
  int nblk;   // 4x4 blocks in the lower triangle incl. diagonal
  __host__ __device__ size_t z_floats() const { return static_cast<size_t>(S) * Fpad * LD; }
};

__host__ __device__ inline Tile make_tile(int T, int D, int S) {
  Tile tl;
  tl.S = S;
  tl.F = T + 1;
  tl.Fpad = (tl.F + 3) & ~3;
  tl.LD = D + 4;
  const int nb = tl.Fpad / 4;
  tl.nblk = nb * (nb + 1) / 2;
  return tl;
}

__device__ __forceinline__ void interact_from_lds(const float* Zall, const Tile& tl, int D, int b0, int B,
                                                  float* __restrict__ out_inter) {
  const int W = D + tl.F * (tl.F - 1) / 2;
  const int items = tl.S * tl.nblk;
  for (int w = threadIdx.x; w < items; w += kThreads) {
    const int s = w / tl.nblk, blk = w - s * tl.nblk;
    const int b = b0 + s;
    if (b >= B) continue;
    int bi, bj;
    block_pair(blk, bi, bj);
    dots_block(Zall + static_cast<size_t>(s) * tl.Fpad * tl.LD, tl.F, D, tl.LD, bi, bj,
               out_inter + static_cast<size_t>(b) * W + D);
  }
}

// ---------------------------------------------------------------------------
// fused forward: gather + pool into LDS, e0, dots, write [e0 | dots]
// ---------------------------------------------------------------------------
template <int DT, int LPR>
__global__ __launch_bounds__(kThreads) void fused_kernel(FwdArgs a, int S) {
  using G = GatherShape<DT, LPR>;
  constexpr int NB = kBagsPerWave;
  extern __shared__ __align__(16) float smem[];
  const Tile tl = make_tile(a.T, a.D, S);
  float* Z = smem;
  int* offs = reinterpret_cast<int*>(smem + tl.z_floats());  // [T][S+1]
  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int b0 = lb * S;
  const int T = a.T, B = a.B, D = a.D;
  const int W = D + tl.F * (tl.F - 1) / 2;

  for (int i = threadIdx.x; i < T * (S + 1); i += kThreads) {
    const int t = i / (S + 1), j = i - t * (S + 1);
    const int b = min(b0 + j, B);
    offs[i] = a.offsets[t * B + b];
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int nbags = S * T;
  for (int j0 = wave * NB; j0 < nbags; j0 += kWavesPerBlock * NB) {
    int t[NB], begin[NB], n[NB], sm[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int j = j0 + k;
      t[k] = 0; begin[k] = 0; n[k] = 0; sm[k] = -1;
      if (j < nbags) {
        const int s = j / T, tt = j - s * T;
        if (b0 + s < B) {
          int s0 = offs[tt * (S + 1) + s], s1 = offs[tt * (S + 1) + s + 1];
          check_range(tt, b0 + s, T, B, a.nnz, s0, s1, a.status);
          t[k] = tt; sm[k] = s;
          begin[k] = __builtin_amdgcn_readfirstlane(s0);
          n[k] = __builtin_amdgcn_readfirstlane(s1 - s0);
        }
      }
    }
    float acc[NB][G::EL];
    gather_bags<DT, LPR, NB>(a.tabs, a.indices, t, begin, n, acc, a.status);
    if (lane < LPR) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (sm[k] < 0) continue;
        float* z = Z + (static_cast<size_t>(sm[k]) * tl.Fpad + 1 + t[k]) * tl.LD + lane * G::EL;
#pragma unroll
        for (int e = 0; e < G::EL; e += 4)
          *reinterpret_cast<float4*>(z + e) = make_float4(acc[k][e], acc[k][e + 1], acc[k][e + 2], acc[k][e + 3]);
        if (a.out_pooled) {
          float* o = a.out_pooled + (static_cast<size_t>(b0 + sm[k]) * T + t[k]) * D + lane * G::EL;
#pragma unroll
          for (int e = 0; e < G::EL; e += 4)
            *reinterpret_cast<float4*>(o + e) = make_float4(acc[k][e], acc[k][e + 1], acc[k][e + 2], acc[k][e + 3]);
        }
      }
    }
  }
  for (int i = threadIdx.x; i < S * D; i += kThreads) {
    const int s = i / D, d = i - s * D;
    const int b = b0 + s;
    if (b < B) {
      const float v = a.e0[static_cast<size_t>(b) * D + d];
      Z[static_cast<size_t>(s) * tl.Fpad * tl.LD + d] = v;
      store_stream(a.out_inter + static_cast<size_t>(b) * W + d, v);
    }
  }
  __syncthreads();
  interact_from_lds(Z, tl, D, b0, B, a.out_inter);
}

// ---------------------------------------------------------------------------
// standalone interaction: Z from pooled + e0 in HBM
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void interact_kernel(int T, int B, int D, const float* __restrict__ e0,
                                                            const float* __restrict__ pooled,
                                                            float* __restrict__ out, int S) {
  extern __shared__ __align__(16) float smem[];
  const Tile tl = make_tile(T, D, S);
  const int b0 = xcd_block(blockIdx.x, gridDim.x) * S;
  const int W = D + tl.F * (tl.F - 1) / 2;
  const int D4 = D / 4;
  for (int i = threadIdx.x; i < S * tl.F * D4; i += kThreads) {
    const int s = i / (tl.F * D4);
    const int rem = i - s * tl.F * D4;
    const int f = rem / D4, d = (rem - f * D4) * 4;
    const int b = b0 + s;
    if (b >= B) continue;
    float4 v;
    if (f == 0) {
      v = *reinterpret_cast<const float4*>(e0 + static_cast<size_t>(b) * D + d);
      float* o = out + static_cast<size_t>(b) * W + d;
      store_stream(o + 0, v.x); store_stream(o + 1, v.y); store_stream(o + 2, v.z); store_stream(o + 3, v.w);
    } else {
      v = *reinterpret_cast<const float4*>(pooled + (static_cast<size_t>(b) * T + (f - 1)) * D + d);
    }
    *reinterpret_cast<float4*>(smem + (static_cast<size_t>(s) * tl.Fpad + f) * tl.LD + d) = v;
  }
  __syncthreads();
  interact_from_lds(smem, tl, D, b0, B, out);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int fwd_supported_row_bytes(int D, int dtype) {
  const int s = dtype == DLRM_F32 ? 4 : 2;
  const long rb = static_cast<long>(D) * s;
  if (rb < 16 || rb > 1024 || (rb & (rb - 1)) != 0) return 0;
  return static_cast<int>(rb);
}

static constexpr size_t kMaxLds = 160 * 1024;

static int pick_samples_per_block(int T, int B, int D) {
  int S = 1;
  while (S * T < 16 && S < B) S *= 2;  // at least ~16 bags per workgroup
  for (;;) {
    const Tile tl = make_tile(T, D, S);
    const size_t lds = tl.z_floats() * 4 + static_cast<size_t>(T) * (S + 1) * 4;
    if (lds <= kMaxLds / 2 || S == 1) return S;
    S /= 2;
  }
}

template <int DT, int LPR>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  if (a.out_inter) {
    const int S = pick_samples_per_block(a.T, a.B, a.D);
    const Tile tl = make_tile(a.T, a.D, S);
    const size_t lds = tl.z_floats() * 4 + static_cast<size_t>(a.T) * (S + 1) * 4;
    if (lds > kMaxLds) return hipErrorInvalidValue;
    const int grid = (a.B + S - 1) / S;
    hipLaunchKernelGGL((fused_kernel<DT, LPR>), dim3(grid), dim3(kThreads), lds, st, a, S);
  } else {
    const long pairs = (static_cast<long>(a.T) * a.B + kBagsPerWave - 1) / kBagsPerWave;
    long grid = (pairs + kWavesPerBlock - 1) / kWavesPerBlock;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL((pool_kernel<DT, LPR>), dim3(static_cast<int>(grid)), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_fwd_dt(const FwdArgs& a, hipStream_t st) {
  switch (fwd_supported_row_bytes(a.D, a.dtype) / 16) {
    case 1: return launch_fwd_t<DT, 1>(a, st);
    case 2: return launch_fwd_t<DT, 2>(a, st);
    case 4: return launch_fwd_t<DT, 4>(a, st);
    case 8: return launch_fwd_t<DT, 8>(a, st);
    case 16: return launch_fwd_t<DT, 16>(a, st);
    case 32: return launch_fwd_t<DT, 32>(a, st);
    case 64: return launch_fwd_t<DT, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_embbag_fwd(const FwdArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case DLRM_F32: return launch_fwd_dt<DLRM_F32>(a, st);
    case DLRM_F16: return launch_fwd_dt<DLRM_F16>(a, st);
    case DLRM_BF16: return launch_fwd_dt<DLRM_BF16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_interact(int T, int B, int D, const float* e0, const float* pooled, float* out, hipStream_t st) {
  int S = 1;
  while (S * (T + 1) < 16 && S < B) S *= 2;
  for (;;) {
    const Tile tl = make_tile(T, D, S);
    if (tl.z_floats() * 4 <= kMaxLds / 2 || S == 1) break;
    S /= 2;
  }
  const Tile tl = make_tile(T, D, S);
  const size_t lds = tl.z_floats() * 4;
  if (lds > kMaxLds) return hipErrorInvalidValue;
  const int grid = (B + S - 1) / S;
  hipLaunchKernelGGL(interact_kernel, dim3(grid), dim3(kThreads), lds, st, T, B, D, e0, pooled, out, S);
  return hipGetLastError();
}

}  // namespace dlrm
