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

// Z: [Fpad][LD] fp32 in LDS (rows >= F may hold anything). The 16 lanes of a
// group (l = 0..15) compute the dots of block (bi, bj): rows i = 4bi..4bi+3
// against rows j = 4bj..4bj+3. Lane l sums the float4 column chunks l, l+16,
// l+32, ... of the block's eight rows; a 4-step exchange (lane distances 8, 4,
// 2, 1, each step halving the values a lane keeps) then leaves lane l with the
// complete dot of pair (4bi + l/4, 4bj + l%4). Pairs j < i < F go to
// out[i(i-1)/2 + j]; with self-pairs, j <= i < F go to out[i(i+1)/2 + j]. Dots
// of rows >= F stay in their own lanes and are dropped. The 16 lanes must run
// this together (every exchange reads an active lane).
template <bool TO_LDS>
__device__ __forceinline__ void dots_block16(const float* Z, int F, int D, int LD, int bi, int bj, int l,
                                             float* __restrict__ out, bool self_pairs = false) {
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.f;
  const float* zi = Z + 4 * bi * LD;
  const float* zj = Z + 4 * bj * LD;
  for (int d = 4 * l; d < D; d += 64) {
    float4 x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = *reinterpret_cast<const float4*>(zi + r * LD + d);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 y = *reinterpret_cast<const float4*>(zj + q * LD + d);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float t = acc[4 * r + q];
        t = fmaf(x[r].x, y.x, t);
        t = fmaf(x[r].y, y.y, t);
        t = fmaf(x[r].z, y.z, t);
        t = fmaf(x[r].w, y.w, t);
        acc[4 * r + q] = t;
      }
    }
  }
  // keep the half of the values whose index has bit k equal to the lane's bit
  // k, and add the partner's copy of that half
  float v8[8], v4[4], v2[2];
  const bool h3 = l & 8, h2 = l & 4, h1 = l & 2, h0 = l & 1;
#pragma unroll
  for (int m = 0; m < 8; ++m) v8[m] = (h3 ? acc[m + 8] : acc[m]) + __shfl_xor(h3 ? acc[m] : acc[m + 8], 8, kWave);
#pragma unroll
  for (int m = 0; m < 4; ++m) v4[m] = (h2 ? v8[m + 4] : v8[m]) + __shfl_xor(h2 ? v8[m] : v8[m + 4], 4, kWave);
#pragma unroll
  for (int m = 0; m < 2; ++m) v2[m] = (h1 ? v4[m + 2] : v4[m]) + __shfl_xor(h1 ? v4[m] : v4[m + 2], 2, kWave);
  const float dot = (h0 ? v2[1] : v2[0]) + __shfl_xor(h0 ? v2[0] : v2[1], 1, kWave);
  const int i = 4 * bi + (l >> 2), j = 4 * bj + (l & 3);
  if (i < F && (j < i || (self_pairs && j == i))) {
    const int k = self_pairs ? i * (i + 1) / 2 + j : i * (i - 1) / 2 + j;
    if constexpr (TO_LDS) out[k] = dot;
    else store_stream(out + k, dot);
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

// Dots of the workgroup's samples into out_inter; with with_emb the dots of a
// sample start after its F Z rows (written by the caller), else after e0.
__device__ __forceinline__ void interact_from_lds(const float* Zall, const Tile& tl, int D, int b0, int B,
                                                  float* __restrict__ out_inter, bool self_pairs, bool with_emb) {
  const int dot0 = with_emb ? tl.F * D : D;
  const int W = dot0 + (self_pairs ? tl.F * (tl.F + 1) / 2 : tl.F * (tl.F - 1) / 2);
  const int items = tl.S * tl.nblk;
  const int l = threadIdx.x & 15;
  for (int w = threadIdx.x >> 4; w < items; w += kThreads / 16) {  // one 4x4 block per 16 lanes
    const int s = w / tl.nblk, blk = w - s * tl.nblk;
    const int b = b0 + s;
    if (b >= B) continue;
    int bi, bj;
    block_pair(blk, bi, bj);
    dots_block16<false>(Zall + static_cast<size_t>(s) * tl.Fpad * tl.LD, tl.F, D, tl.LD, bi, bj, l,
                        out_inter + static_cast<size_t>(b) * W + dot0, self_pairs);
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
  const bool self_pairs = (a.layout & DLRM_PAIRS_SELF) != 0;
  const bool with_emb = (a.layout & DLRM_WITH_EMBEDDINGS) != 0;
  const int W = (with_emb ? tl.F * D : D) + (self_pairs ? tl.F * (tl.F + 1) / 2 : tl.F * (tl.F - 1) / 2);

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
      if (!with_emb) store_stream(a.out_inter + static_cast<size_t>(b) * W + d, v);
    }
  }
  __syncthreads();
  if (with_emb) {  // the F Z rows of every sample ahead of its dots
    for (int i = threadIdx.x; i < S * tl.F * D; i += kThreads) {
      const int s = i / (tl.F * D), r = i - s * tl.F * D;
      const int f = r / D, d = r - f * D;
      const int b = b0 + s;
      if (b < B) store_stream(a.out_inter + static_cast<size_t>(b) * W + r,
                              Z[(static_cast<size_t>(s) * tl.Fpad + f) * tl.LD + d]);
    }
  }
  interact_from_lds(Z, tl, D, b0, B, a.out_inter, self_pairs, with_emb);
}

// ---------------------------------------------------------------------------
// standalone interaction: Z from pooled + e0 in HBM
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void interact_kernel(int T, int B, int D, const float* __restrict__ e0,
                                                            const float* __restrict__ pooled,
                                                            float* __restrict__ out, int S, int layout) {
  extern __shared__ __align__(16) float smem[];
  const Tile tl = make_tile(T, D, S);
  const int b0 = xcd_block(blockIdx.x, gridDim.x) * S;
  const bool self_pairs = (layout & DLRM_PAIRS_SELF) != 0;
  const bool with_emb = (layout & DLRM_WITH_EMBEDDINGS) != 0;
  const int W = (with_emb ? tl.F * D : D) + (self_pairs ? tl.F * (tl.F + 1) / 2 : tl.F * (tl.F - 1) / 2);
  const int D4 = D / 4;
  for (int i = threadIdx.x; i < S * tl.F * D4; i += kThreads) {
    const int s = i / (tl.F * D4);
    const int rem = i - s * tl.F * D4;
    const int f = rem / D4, d = (rem - f * D4) * 4;
    const int b = b0 + s;
    if (b >= B) continue;
    float4 v;
    if (f == 0) v = *reinterpret_cast<const float4*>(e0 + static_cast<size_t>(b) * D + d);
    else v = *reinterpret_cast<const float4*>(pooled + (static_cast<size_t>(b) * T + (f - 1)) * D + d);
    if (f == 0 || with_emb) {  // e0 (and with with_emb every Z row) ahead of the dots
      float* o = out + static_cast<size_t>(b) * W + f * D + d;
      store_stream(o + 0, v.x); store_stream(o + 1, v.y); store_stream(o + 2, v.z); store_stream(o + 3, v.w);
    }
    *reinterpret_cast<float4*>(smem + (static_cast<size_t>(s) * tl.Fpad + f) * tl.LD + d) = v;
  }
  __syncthreads();
  interact_from_lds(smem, tl, D, b0, B, out, self_pairs, with_emb);
}

// ---------------------------------------------------------------------------
// row-streaming fused forward: one sample per 512-thread workgroup
// ---------------------------------------------------------------------------
// For rows of 128..1024 bytes, one wave-wide load fetches exactly one table row
// (LB = row bytes / 64 per lane), so a wave can stream the rows of consecutive
// bags without any cross-lane reduction: every lane owns the same EL columns of
// every row. The sample's bags are laid end to end into one row stream whose
// indices are staged in LDS up front (one round trip for all of them); the 8
// waves split the stream into equal contiguous ranges, keep WIN row loads in
// flight, and sum rows in stream order. A bag cut by a range boundary is
// finished by adding the later waves' partial sums in wave order after a
// barrier, so the result does not depend on timing.
//
// Interaction: with T >= 24 the Gram matrix of Z is a real dense contraction
// and runs on MFMA. For 16-bit and quantized tables the dots of e0 with each
// pooled row are taken in fp32 and the Gram of the pooled rows in 16x16 tiles
// (16x16x32 bf16), each operand split into bf16 hi + lo in registers as it is
// read from LDS (hi*hi + hi*lo + lo*hi in fp32); for fp32 tables the whole
// Gram in 32x32 tiles (32x32x16 bf16) with a three-way split. Otherwise 4x4
// register blocks of fp32 FMAs. The output row is assembled in LDS and written
// with contiguous stores.
constexpr int kRowThreads = 512;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kStageCap = 2048;  // staged indices per sample; longer streams read indices from HBM

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// Global (not generic) pointers.
template <class T>
using gptr = const __attribute__((address_space(1))) T*;

// Buffer resource of one table row (or output row): base = its address
// (wave-uniform), num_records = the bytes the lanes may touch. A window slot
// that reads nothing (past the range, or an index outside its table) gets 0:
// every lane is then out of range, the load returns zeros and makes no memory
// request, so padding slots cost no traffic. (With global loads of a fixed
// fallback row instead, the multi-hot batch of 8 fp16 tables took 29.6 us
// against 27.7 us.) Word 3 is the raw-buffer configuration for gfx950.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(uint64_t row, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(row), 0, nbytes, 0x00020000);
}
// Row loads are non-temporal: without it the capacity batch (64 tables of
// 10M bf16 rows of 256 bytes, 16384 samples) takes 824 us instead of 772 us.
constexpr int kNonTemporal = 2;
// Output stores at system scope (sc0 sc1): each wave's store is written on to
// memory as it arrives instead of leaving dirty lines for later eviction
// between the random row reads. Capacity batch: 771 us, against 784 us with
// non-temporal global stores and 801 us with plain ones.
constexpr int kStoreSystem = 17;
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t r, int i, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, i * 4, 0, kStoreSystem);
}

template <int LB>
struct LaneChunk;
template <>
struct LaneChunk<1> {
  using type = uint32_t;  // low 8 bits used
  __device__ static type bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, kNonTemporal);
  }
  __device__ static type zero() { return 0u; }
};
template <>
struct LaneChunk<2> {
  using type = uint32_t;  // low 16 bits used
  __device__ static type bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kNonTemporal);
  }
  __device__ static type zero() { return 0u; }
};
template <>
struct LaneChunk<4> {
  using type = uint32_t;
  __device__ static type bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNonTemporal);
  }
  __device__ static type zero() { return 0u; }
};
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <>
struct LaneChunk<8> {
  using type = uint2;
  __device__ static type bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNonTemporal);
    return make_uint2(v.x, v.y);
  }
  __device__ static type zero() { return make_uint2(0u, 0u); }
};
template <>
struct LaneChunk<16> {
  using type = uint4;
  __device__ static type bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ static type zero() { return make_uint4(0u, 0u, 0u, 0u); }
};

// Broadcast lane j's 64-bit value (two 32-bit halves) to a scalar.
__device__ __forceinline__ uint64_t bcast64(uint32_t lo, uint32_t hi, int j) {
  const uint32_t l = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), j));
  const uint32_t h = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), j));
  return (static_cast<uint64_t>(h) << 32) | l;
}

template <int DT>
__device__ __forceinline__ float decode_lo(uint32_t w) {
  if constexpr (DT == DLRM_BF16) return bf16_lo(w);
  else if constexpr (DT == DLRM_F16) return f16_lo(w);
  else return __uint_as_float(w);
}
template <int DT>
__device__ __forceinline__ float decode_hi(uint32_t w) {
  if constexpr (DT == DLRM_BF16) return bf16_hi(w);
  else return f16_hi(w);
}

// acc[0..EL) += the lane's part of one row.
template <int DT, int LB>
__device__ __forceinline__ void acc_chunk(float* acc, const typename LaneChunk<LB>::type& v) {
  if constexpr (LB == 2) {
    acc[0] += decode_lo<DT>(v);
  } else if constexpr (LB == 4) {
    if constexpr (DT == DLRM_F32) acc[0] += __uint_as_float(v);
    else { acc[0] += decode_lo<DT>(v); acc[1] += decode_hi<DT>(v); }
  } else if constexpr (LB == 8) {
    if constexpr (DT == DLRM_F32) { acc[0] += __uint_as_float(v.x); acc[1] += __uint_as_float(v.y); }
    else {
      acc[0] += decode_lo<DT>(v.x); acc[1] += decode_hi<DT>(v.x);
      acc[2] += decode_lo<DT>(v.y); acc[3] += decode_hi<DT>(v.y);
    }
  } else {
    accumulate16<DT>(acc, v);
  }
}

// Table-wise 8-bit rows: acc[0..LB) += s * q for the lane's LB codes q (uint8).
__device__ __forceinline__ float ubyte(uint32_t w, int k) { return static_cast<float>((w >> (8 * k)) & 0xffu); }

template <int LB>
__device__ __forceinline__ void acc_chunk_q8(float* acc, const typename LaneChunk<LB>::type& v, float s) {
  if constexpr (LB == 2) {
    acc[0] = fmaf(s, ubyte(v, 0), acc[0]);
    acc[1] = fmaf(s, ubyte(v, 1), acc[1]);
  } else if constexpr (LB == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = fmaf(s, ubyte(v, k), acc[k]);
  } else {
    static_assert(LB == 8, "8-bit rows of 128, 256 or 512 bytes");
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[k] = fmaf(s, ubyte(v.x, k), acc[k]);
      acc[4 + k] = fmaf(s, ubyte(v.y, k), acc[4 + k]);
    }
  }
}

// Row-wise 4-bit rows: the lane's LB code bytes hold 2 LB columns, byte k the
// column 2k in its low nibble and 2k + 1 in its high nibble;
// acc[0..2 LB) += s * q.
__device__ __forceinline__ float nibble(uint32_t w, int k) { return static_cast<float>((w >> (4 * k)) & 0xfu); }

template <int LB>
__device__ __forceinline__ void acc_chunk_q4(float* acc, const typename LaneChunk<LB>::type& v, float s) {
  if constexpr (LB == 1) {
    acc[0] = fmaf(s, nibble(v, 0), acc[0]);
    acc[1] = fmaf(s, nibble(v, 1), acc[1]);
  } else if constexpr (LB == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = fmaf(s, nibble(v, k), acc[k]);
  } else {
    static_assert(LB == 4, "4-bit codes of 64, 128 or 256 bytes per row");
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(s, nibble(v, k), acc[k]);
  }
}

// Bytes from one row-wise 4-bit row to the next: the code bytes and the fp32
// (scale, bias) pair, rounded up to a power of two so that a row never
// straddles more lines than its size needs (one 128-byte line for 128 columns).
__host__ __device__ constexpr int q4_row_stride(int code_bytes) {
  int s = 16;
  while (s < code_bytes + 8) s *= 2;
  return s;
}

template <int DT, int LB>
struct RowShape {
  static constexpr int EL = DT == DLRM_Q4 ? 2 * LB : LB / Storage<DT>::bytes;  // fp32 columns per lane
  // rows per window (two windows in flight: 32 VGPRs); 8-bit rows also carry a
  // scale and a bias per row and keep more columns per lane, so their windows
  // are smaller
  // (16-bit rows of 512 and 1024 bytes and table-wise 8-bit rows keep a few
  // rows fewer in flight, which keeps them within 80 VGPRs without spills;
  // bf16 rows of 256 bytes keep 12: on the 64-table capacity batch 12, 16 and
  // 20 rows per window measured 780.5, 784.8 and 793.3 us, bit-identical;
  // fp32 rows of 512 bytes keep 7, so that a 26-row sample split over two
  // waves is gathered in one round trip per wave: 17.1 us against 17.6 us
  // with 6 on the 26-table batch; 128-byte 16-bit rows keep 16: 12 measured
  // 27.7 us against 27.3 us on the multi-hot batch)
  static constexpr int WIN = DT == DLRM_Q4                   ? (LB >= 4 ? 6 : 12)
                             : DT == DLRM_Q8T                ? (LB >= 8 ? 4 : 12)
                             : (DT != DLRM_F32 && LB == 16) ? 3
                             : (DT != DLRM_F32 && LB == 8)  ? 6
                             : (DT == DLRM_BF16 && LB == 4) ? 12
                             : (DT == DLRM_F32 && LB == 8)  ? 7
                                                             : (LB >= 4 ? 64 / LB : 16);
};

// LDS of the row-streaming kernel: table bases, row counts and 8-bit scales
// shared by the workgroup, then G identical per-group regions (a group of
// 512/G threads works on its own sample). Offsets marked "in a group" are
// relative to the group's region.
struct RowLayout {
  int G;         // sample groups per workgroup (1, 2, 4, 8)
  int Tp;        // Z rows after e0 (T rounded up: 32 for MFMA, else to F multiple of 4)
  int LD;        // Z row stride in floats
  int off_tbase;
  int off_trows;
  int off_qsb;   // table-wise 8-bit rows: (scale, bias) per table
  int off_groups;
  int group_bytes;
  // in a group:
  int off_beg;   // bag tables, double-buffered
  int off_pos;
  int pos_stride;  // bytes between the two bag-table buffers
  int off_carry_t;
  int off_stage;
  int off_sbag;
  int off_carry;
  int off_out;
  int off_z;
  int bytes;
};

__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }

__host__ __device__ inline RowLayout make_row_layout(int T, int D, bool mfma, int G = 1) {
  RowLayout L;
  L.G = G;
  L.Tp = mfma ? ((T + 31) / 32) * 32 : (((T + 1 + 3) & ~3) - 1);
  L.LD = D + 4;
  const int P = (T + 1) * (T + 2) / 2;  // dots with self-pairs, the most any layout stages
  int o = 0;
  L.off_tbase = o; o += align16(T * 8);
  L.off_trows = o; o += align16(T * 4);
  L.off_qsb = o; o += align16(T * 8);
  L.off_groups = o;
  const int gw = kRowWaves / G;
  const int cap = kStageCap / G;
  int g = 0;
  L.pos_stride = align16(T * 4) + align16((T + 1) * 4);
  L.off_beg = g;                       // [2] x { bag begin (index position) [T]; stream start [T+1] }
  L.off_pos = g + align16(T * 4);
  g += 2 * L.pos_stride;
  L.off_carry_t = g; g += align16(gw * 4);
  const int uni = g;                   // union { stage + bag ids + carries ; output staging }
  L.off_stage = uni;
  L.off_sbag = L.off_stage + cap * 4;
  L.off_carry = L.off_sbag + align16(cap);
  const int gather_bytes = L.off_carry + gw * D * 4 - uni;
  L.off_out = uni;
  const int out_bytes = (D + P) * 4;
  g = uni + align16(gather_bytes > out_bytes ? gather_bytes : out_bytes);
  L.off_z = g; g += (1 + L.Tp) * L.LD * 4;
  L.group_bytes = align16(g);
  L.bytes = L.off_groups + G * L.group_bytes;
  return L;
}

__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Split 8 fp32 into bf16 hi (round to nearest even) and the bf16 of the
// remainder (x - hi, also rounded to nearest even): x = hi + lo + O(2^-17 |x|).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void split2(float x0, float x1, uint32_t& h, uint32_t& l) {
  const float2_t x = {x0, x1};
  h = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
  const float2_t r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)};
  l = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
}

__device__ __forceinline__ void split_bf16x8(const float4& a, const float4& b, bf16x8_t& hi, bf16x8_t& lo) {
  uint4 h, l;
  split2(a.x, a.y, h.x, l.x);
  split2(a.z, a.w, h.y, l.y);
  split2(b.x, b.y, h.z, l.z);
  split2(b.z, b.w, h.w, l.w);
  hi = __builtin_bit_cast(bf16x8_t, h);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

typedef float floatx4_t __attribute__((ext_vector_type(4)));

// 8 consecutive fp32 values of a Z row in LDS, split in registers into bf16
// hi and lo parts.
__device__ __forceinline__ void load_split8(const float* p, bf16x8_t& hi, bf16x8_t& lo) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  const float4 y = *reinterpret_cast<const float4*>(p + 4);
  split_bf16x8(x, y, hi, lo);
}

// One 16x16 tile (I, J), I >= J, of the Gram matrix of the pooled rows (Z
// rows 1..Tp, fp32 in LDS): hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16
// with fp32 accumulation. Lane l supplies row l % 16 of each block at the 8
// columns 8 (l / 16) .. +8 of every 32-column step (the same columns for both
// operands), and receives the Gram entries of rows 4 (l / 16) .. +4 of block I
// with row l % 16 of block J. Entries with Z-row indices zi > zj (zi >= zj for
// self-pairs), zi <= T, go to dots[zi(zi-1)/2 + zj] (dots[zi(zi+1)/2 + zj]).
__device__ __forceinline__ void gram_tile16(const float* Z, int LD, int D, int T, int I, int J,
                                            float* __restrict__ dots, bool self_pairs, int lane) {
  const int m = lane & 15, kq = lane >> 4;
  const float* za = Z + (1 + 16 * I + m) * LD + 8 * kq;
  const float* zb = Z + (1 + 16 * J + m) * LD + 8 * kq;
  floatx4_t acc = {};
  for (int k0 = 0; k0 < D; k0 += 32) {
    bf16x8_t ah, al, bh, bl;
    load_split8(za + k0, ah, al);
    load_split8(zb + k0, bh, bl);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int zi = 1 + 16 * I + 4 * kq + v, zj = 1 + 16 * J + m;
    if (zi <= T && (zi > zj || (self_pairs && zi == zj)))
      dots[self_pairs ? zi * (zi + 1) / 2 + zj : zi * (zi - 1) / 2 + zj] = acc[v];
  }
}

// Three-way split of 2 fp32 values into bf16 parts: x = h + m + l up to
// 2^-27 |x| (h = bf16(x), m = bf16(x - h), l = bf16(x - h - m); both
// differences are exact in fp32).
__device__ __forceinline__ void split3(float x0, float x1, uint32_t& h, uint32_t& m, uint32_t& l) {
  const float2_t x = {x0, x1};
  h = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
  const float2_t r1 = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)};
  m = __builtin_bit_cast(uint32_t, __builtin_convertvector(r1, bf16x2_t));
  const float2_t r2 = {r1[0] - __uint_as_float(m << 16), r1[1] - __uint_as_float(m & 0xffff0000u)};
  l = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2_t));
}

__device__ __forceinline__ void load_split3x8(const float* p, bf16x8_t& h, bf16x8_t& m, bf16x8_t& l) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  const float4 y = *reinterpret_cast<const float4*>(p + 4);
  uint4 uh, um, ul;
  split3(x.x, x.y, uh.x, um.x, ul.x);
  split3(x.z, x.w, uh.y, um.y, ul.y);
  split3(y.x, y.y, uh.z, um.z, ul.z);
  split3(y.z, y.w, uh.w, um.w, ul.w);
  h = __builtin_bit_cast(bf16x8_t, uh);
  m = __builtin_bit_cast(bf16x8_t, um);
  l = __builtin_bit_cast(bf16x8_t, ul);
}

// One 32x32 tile (I, J), I >= J, of the Gram matrix of every Z row (e0 and
// the pooled rows, fp32 in LDS) for fp32 tables, on v_mfma_f32_32x32x16_bf16
// with each operand split three ways (hi, mid, lo) in registers: the products
// hh + hm + mh + hl + lh + mm (taken smallest first) leave out terms below
// 5 * 2^-27 |a||b|, so the dots keep fp32 accuracy. Lane l supplies row
// l % 32 of each block at the 8 columns 8 (l / 32) .. +8 of every 16-column
// step and receives rows 8 (v / 4) + 4 (l / 32) + v % 4 (v = 0..15) of block I
// with row l % 32 of block J. A diagonal tile reads and splits its rows once
// for both operands. Rows past the last Z row read that row (their entries are
// dropped), so Z needs no padding rows.
__device__ __forceinline__ void gram_tile32_x6(const float* Z, int LD, int D, int F, int I, int J,
                                               float* __restrict__ dots, bool self_pairs, int lane) {
  const int m = lane & 31, kq = lane >> 5;
  const int ra = min(32 * I + m, F - 1), rb = min(32 * J + m, F - 1);
  const float* za = Z + ra * LD + 8 * kq;
  const float* zb = Z + rb * LD + 8 * kq;
  floatx16_t acc = {};
  for (int k0 = 0; k0 < D; k0 += 16) {
    bf16x8_t ah, am, al, bh, bm, bl;
    load_split3x8(za + k0, ah, am, al);
    if (I == J) {
      bh = ah;
      bm = am;
      bl = al;
    } else {
      load_split3x8(zb + k0, bh, bm, bl);
    }
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bm, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bm, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int zi = 32 * I + 8 * (v >> 2) + 4 * kq + (v & 3), zj = 32 * J + m;
    if (zi < F && (zi > zj || (self_pairs && zi == zj)))
      dots[self_pairs ? zi * (zi + 1) / 2 + zj : zi * (zi - 1) / 2 + zj] = acc[v];
  }
}

// Dots of e0 (Z row 0) with every pooled row (and with itself for
// self-pairs), in fp32: 8 lanes per dot, lane j over the float4 chunks j, j+8,
// ... of D, combined in a fixed order. Pair (zi, 0) sits at out[zi(zi-1)/2]
// (out[zi(zi+1)/2] with self-pairs), out being the start of the dots.
template <int NT>
__device__ __forceinline__ void e0_dots(const float* Z, int LD, int D, int T, float* out, int tid,
                                        bool self_pairs) {
  const int j = tid & 7;
  for (int zi = (self_pairs ? 0 : 1) + (tid >> 3); zi <= T; zi += NT / 8) {
    const float* zr = Z + zi * LD;
    float sum = 0.f;
    for (int d = 4 * j; d < D; d += 32) {
      const float4 x = *reinterpret_cast<const float4*>(zr + d);
      const float4 y = *reinterpret_cast<const float4*>(Z + d);
      sum = fmaf(x.x, y.x, sum);
      sum = fmaf(x.y, y.y, sum);
      sum = fmaf(x.z, y.z, sum);
      sum = fmaf(x.w, y.w, sum);
    }
    sum += __shfl_xor(sum, 1, kWave);
    sum += __shfl_xor(sum, 2, kWave);
    sum += __shfl_xor(sum, 4, kWave);
    if (j == 0) out[self_pairs ? zi * (zi + 1) / 2 : zi * (zi - 1) / 2] = sum;
  }
}

// Per-window state: each lane's row address (as two halves) and bag, and the
// wave-wide masks of rows that end a partial sum and rows that must be skipped.
struct Window {
  uint32_t alo, ahi;
  int tk;
  unsigned long long fmask, smask;
  float sc, bi;  // 8-bit rows: this lane's row's scale and bias (in flight with the rows)
};

struct RowCursor {
  bool to_carry;  // the next flushed sum continues a bag begun by an earlier wave
};

// Largest t in [0, T) with pos[t] <= x, for non-decreasing pos with pos[0] <=
// x: the bag (skipping empty ones) that holds stream position x. A fixed
// number of halving steps, each one LDS read, so that independent searches of
// one thread overlap instead of running as data-dependent loops.
__device__ __forceinline__ int last_le(const int* pos, int T, int x) {
  static_assert(DLRM_MAX_TABLES <= 128, "steps below cover T <= 128");
  int lo = 0;
#pragma unroll
  for (int step = 64; step > 0; step >>= 1) {
    const int c = lo + step;
    const int v = pos[c < T ? c : T - 1];
    if (c < T && v <= x) lo = c;
  }
  return lo;
}

// BEYOND: the range may reach past the staged positions (a sample of more than
// kStageCap rows); only then does this read indices from HBM. Keeping that
// path out of the common loop keeps the loop free of loads other than the
// table rows, so the compiler's wait counts stay exact.
// 8-bit rows. QM = 1 (row-wise): D codes followed by the row's fp32 scale and
// bias, rows RB + 8 bytes apart; each lane also loads the (scale, bias) pair of
// "its" row of the window. QM = 2 (table-wise): D codes per row, the table's
// (scale, bias) pair read from LDS (qsb).
template <int WIN, int RB, bool BEYOND, int QM, int CAP>
__device__ __forceinline__ void prepare_window(Window& w, const FwdArgs& a, const int* sm_beg, const int* sm_pos,
                                               const int* stage, const uint8_t* sbag, const char* const* tbase,
                                               const int* trows, int T, int q, int p1, uint64_t fallback,
                                               int tid, const float* qsb = nullptr) {
  constexpr uint64_t kStride = QM == 1 ? q4_row_stride(RB) : RB;
  const int lane = tid & (kWave - 1);
  uint64_t addr = fallback;
  int tk = 0;
  bool flush = false, skip = true;
  const int pos = q + lane;
  if (lane < WIN && pos < p1) {
    int r;
    if (!BEYOND || pos < CAP) {
      r = stage[pos];
      tk = sbag[pos];
    } else {  // beyond the staging area: locate the bag and read the index from HBM
      const int lo = last_le(sm_pos, T, pos);
      tk = lo;
      r = a.indices[sm_beg[lo] + (pos - sm_pos[lo])];
      if (r < 0 || r >= trows[lo]) {
        r = -1;
        flag(a.status, DLRM_STATUS_BAD_INDEX);
      }
    }
    if (r >= 0) {  // an index outside its table is skipped (its load reads nothing)
      addr = reinterpret_cast<uint64_t>(tbase[tk]) + static_cast<uint64_t>(r) * kStride;
      skip = false;
    }
    flush = (pos + 1 == sm_pos[tk + 1]) || (pos + 1 == p1);
  }
  if constexpr (QM == 1) {
    // every lane loads the (scale, bias) pair of its row (skipped slots: the fallback row's)
    const auto p = reinterpret_cast<gptr<uint32_t>>(addr + RB);
    w.sc = __uint_as_float(p[0]);
    w.bi = __uint_as_float(p[1]);
  } else if constexpr (QM == 2) {
    w.sc = qsb[2 * tk];
    w.bi = qsb[2 * tk + 1];
  }
  w.alo = static_cast<uint32_t>(addr);
  w.ahi = static_cast<uint32_t>(addr >> 32);
  w.tk = tk;
  constexpr unsigned long long kWinMask = WIN >= 64 ? ~0ull : ((1ull << WIN) - 1);
  w.fmask = __ballot(flush) & kWinMask;
  w.smask = __ballot(skip) & kWinMask;
}

template <class C, int WIN, int RB>
__device__ __forceinline__ void issue_window(const Window& w, typename C::type (&v)[WIN], uint32_t lane_off) {
#pragma unroll
  for (int j = 0; j < WIN; ++j) {
    const int nbytes = ((w.smask >> j) & 1ull) ? 0 : RB;
    v[j] = C::bload(row_rsrc(bcast64(w.alo, w.ahi, j), nbytes), lane_off);
  }
}

template <int DT, int LB, int WIN>
__device__ __forceinline__ void consume_window(const Window& w, typename LaneChunk<LB>::type (&v)[WIN],
                                               float (&acc)[RowShape<DT, LB>::EL], RowCursor& cur, float* Z,
                                               int LD, float* carry_w, int* carry_t_w, int tid, float& bacc) {
  constexpr int EL = RowShape<DT, LB>::EL;
  const int lane = tid & (kWave - 1);
#pragma unroll
  for (int j = 0; j < WIN; ++j) {
    // a skipped slot's load read nothing and returned zeros
    const bool skipped = (w.smask >> j) & 1ull;
    const typename LaneChunk<LB>::type x = v[j];
    if constexpr (DT == DLRM_Q4 || DT == DLRM_Q8T) {
      // scale * q summed per column; the biases of the bag's rows summed once
      const float sj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w.sc), j));
      const float bj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w.bi), j));
      if constexpr (DT == DLRM_Q4) acc_chunk_q4<LB>(acc, x, skipped ? 0.f : sj);
      else acc_chunk_q8<LB>(acc, x, skipped ? 0.f : sj);
      bacc += skipped ? 0.f : bj;
    } else {
      acc_chunk<DT, LB>(acc, x);
    }
    if ((w.fmask >> j) & 1ull) {
      const int tj = __builtin_amdgcn_readlane(w.tk, j);
      float* dst = Z + (1 + tj) * LD;
      if (cur.to_carry) {
        dst = carry_w;
        if (lane == 0) *carry_t_w = tj;
        cur.to_carry = false;
      }
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        dst[lane * EL + e] = (DT == DLRM_Q4 || DT == DLRM_Q8T) ? acc[e] + bacc : acc[e];
        acc[e] = 0.f;
      }
      bacc = 0.f;
    }
  }
}

// Bag (t, b): clamp its CSR range into [0, nnz], report an invalid CSR, and
// publish begin and length for the stream-position scan.
__device__ __forceinline__ void publish_bag(const FwdArgs& a, int t, int b, int s0, int s1, int* beg, int* pos) {
  bool bad = false;
  if (t == 0 && b == 0 && s0 != 0) bad = true;
  if (t == a.T - 1 && b == a.B - 1 && static_cast<int64_t>(s1) != a.nnz) bad = true;
  if (s0 < 0) { s0 = 0; bad = true; }
  if (static_cast<int64_t>(s0) > a.nnz) { s0 = static_cast<int>(a.nnz); bad = true; }
  if (static_cast<int64_t>(s1) > a.nnz) { s1 = static_cast<int>(a.nnz); bad = true; }
  if (s1 < s0) { s1 = s0; bad = true; }
  if (bad) flag(a.status, DLRM_STATUS_BAD_OFFSETS);
  beg[t] = s0;
  pos[t + 1] = s1 - s0;  // a length until scan_positions runs
}

// Z row of an empty bag: no gather writes it, so it is cleared here.
__device__ __forceinline__ void clear_if_empty(const int* pos, int t, float* Z, int LD, int D) {
  if (pos[t + 1] == 0) {
    float* z = Z + (1 + t) * LD;
    for (int d = 0; d < D; d += 4) *reinterpret_cast<float4*>(z + d) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Inclusive scan of the bag lengths into stream start positions (one wave).
__device__ __forceinline__ void scan_positions(int* pos, int T, int tid) {
  const int lane = tid & (kWave - 1);
  int carry_sum = 0;
  for (int t0 = 0; t0 < T; t0 += kWave) {
    const int t = t0 + lane;
    int v = t < T ? pos[t + 1] : 0;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(v, o, kWave);
      if (lane >= o) v += y;
    }
    if (t < T) pos[t + 1] = v + carry_sum;
    carry_sum += __shfl(v, kWave - 1, kWave);
  }
  if (lane == 0) pos[0] = 0;
}

constexpr int kStagePerThread = kStageCap / kRowThreads;  // the same for every group size

// Issue the loads of a sample's staged indices (stream positions tid + k*NT);
// the values are written to LDS later by write_stage. The bag of each
// position is found first (LDS only); then every load is issued without a
// branch, a position past the stream reading an index of the sample instead,
// so that the loads land straight in r[] and nothing waits for them before
// write_stage.
template <int NT>
__device__ __forceinline__ void load_stage(const FwdArgs& a, const int* beg, const int* pos, int T, int N,
                                           int (&r)[kStagePerThread], int (&tb)[kStagePerThread], int tid) {
  int off[kStagePerThread];
  // with no indices at all, the (always valid) offsets array stands in
  const int* src = a.nnz > 0 ? a.indices : a.offsets;
  const int last = a.nnz > 0 ? static_cast<int>(a.nnz) - 1 : 0;
#pragma unroll
  for (int k = 0; k < kStagePerThread; ++k) {
    // a block of positions wholly past the stream (uniform over the group)
    // skips the search and re-reads block 0's index, a line the group reads
    // anyway (26-table batch: 17.1 -> 16.7 us per launch)
    tb[k] = -1;
    off[k] = k > 0 ? off[0] : 0;
    if (k * NT >= N) continue;
    const int p = tid + k * NT;
    const int pc = p < N ? p : N - 1;
    const int lo = last_le(pos, T, pc);
    tb[k] = p < N ? lo : -1;
    const int o = beg[lo] + (pc - pos[lo]);
    off[k] = o < 0 ? 0 : (o > last ? last : o);
  }
#pragma unroll
  for (int k = 0; k < kStagePerThread; ++k) r[k] = src[off[k]];
}

template <int NT>
__device__ __forceinline__ void write_stage(const FwdArgs& a, const int (&r)[kStagePerThread],
                                            const int (&tb)[kStagePerThread], int* stage, uint8_t* sbag,
                                            const int* trows, int tid) {
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kStagePerThread; ++k) {
    if (tb[k] >= 0) {
      int v = r[k];
      if (v < 0 || v >= trows[tb[k]]) { bad = true; v = -1; }
      stage[tid + k * NT] = v;
      sbag[tid + k * NT] = static_cast<uint8_t>(tb[k]);
    }
  }
  if (bad) flag(a.status, DLRM_STATUS_BAD_INDEX);
}

// An empty use of a value in registers: the compiler must have it (and so
// wait for the load that produced it) at this point.
__device__ __forceinline__ void touch(uint32_t x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void touch(uint2 x) { asm volatile("" ::"v"(x.x), "v"(x.y)); }
__device__ __forceinline__ void touch(uint4 x) { asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w)); }

// Sum stream positions [p0, p1) of one wave into Z rows (or the wave's carry
// slot for a bag begun by an earlier wave), in windows of WIN rows: each lane
// first works out the address of "its" row of a window and whether a sum ends
// there; window k+1's loads are issued before window k is summed. Slots past
// the range issue a load that reads nothing and returns zeros, so every window
// issues the same number of loads (and the compiler's wait counts stay exact).
template <int DT, int LB, bool BEYOND, int CAP, int WIN>
__device__ __forceinline__ void gather_range(const FwdArgs& a, const int* beg, const int* pos, const int* stage,
                                             const uint8_t* sbag, const char* const* tbase, const int* trows, int T,
                                             int p0, int p1, float* Z, int LD, float* carry_w, int* carry_t_w,
                                             int tid, const float* qsb) {
  constexpr int QM = DT == DLRM_Q4 ? 1 : (DT == DLRM_Q8T ? 2 : 0);
  using C = LaneChunk<LB>;
  using RS = RowShape<DT, LB>;
  constexpr int EL = RS::EL;
  constexpr int RB = LB * kWave;  // row bytes
  // the bag holding p0 (a search of fixed length: a wave late in the sample
  // would otherwise walk past dozens of bags before its first load)
  const int t0 = rfl(last_le(pos, T, p0));
  RowCursor cur{rfl(pos[t0]) < p0};
  float acc[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) acc[e] = 0.f;
  float bacc = 0.f;
  const uint64_t fallback = reinterpret_cast<uint64_t>(tbase[0]);
  const uint32_t lane_off = static_cast<uint32_t>(tid & (kWave - 1)) * LB;
  Window wa, wb;
  typename C::type va[WIN], vb[WIN];
  prepare_window<WIN, RB, BEYOND, QM, CAP>(wa, a, beg, pos, stage, sbag, tbase, trows, T, p0, p1, fallback, tid, qsb);
  issue_window<C, WIN, RB>(wa, va, lane_off);
  for (int q = p0;;) {
    prepare_window<WIN, RB, BEYOND, QM, CAP>(wb, a, beg, pos, stage, sbag, tbase, trows, T, q + WIN, p1, fallback, tid,
                                        qsb);
    issue_window<C, WIN, RB>(wb, vb, lane_off);
    consume_window<DT, LB, WIN>(wa, va, acc, cur, Z, LD, carry_w, carry_t_w, tid, bacc);
    q += WIN;
    if (q >= p1) break;
    prepare_window<WIN, RB, BEYOND, QM, CAP>(wa, a, beg, pos, stage, sbag, tbase, trows, T, q + WIN, p1, fallback, tid,
                                        qsb);
    issue_window<C, WIN, RB>(wa, va, lane_off);
    consume_window<DT, LB, WIN>(wb, vb, acc, cur, Z, LD, carry_w, carry_t_w, tid, bacc);
    q += WIN;
    if (q >= p1) break;
  }
  // The loop leaves one window of empty loads (past the range) in flight.
  // Reading every window register here makes the compiler wait for them once
  // per range; otherwise the next sample's loop sees those loads as possibly
  // outstanding and guards each reuse of the registers with a full wait, in
  // every iteration.
#pragma unroll
  for (int j = 0; j < WIN; ++j) {
    touch(va[j]);
    touch(vb[j]);
  }
}

// One sample's gather by one wave for 128-byte rows of 16-bit values (D = 64),
// four rows per load instruction: an instruction takes four consecutive rows
// of one bag, one per quarter of the wave (16 lanes, 8 bytes = four columns
// each). The table is then the same for the whole instruction, so the load
// goes through one buffer resource over the table with a row offset per lane;
// a slot past the bag's end or holding an index outside the table reads past
// the buffer (zeros, no memory request). Quarter k sums rows 4m + k of the bag
// in order; at the bag's end each column's four partial sums are added as
// (q0 + q1) + (q2 + q3) and written to the bag's Z row. Lane (k, i) of a
// window of WIN instructions works out instruction q + i's bag and the row
// quarter k loads in it, so an instruction takes its table base with lane
// reads and each quarter's row offset with a row broadcast (no LDS access
// between two loads). Needs T <= 64, the sample staged in LDS and tables of
// fewer than 2^24 rows (under 2^31 bytes). Multi-hot batch (8 fp16 tables of
// 4M rows, 20 rows per bag): 22.0 us against 27.2 us with one row per load.
struct QuadWindow {
  int t;                       // lane i: instruction q + i's bag
  uint32_t roff;               // lane (k, i): byte offset of the row quarter k loads in instruction q + i
  uint32_t blo, bhi;           // lane i: the bag's table base
  unsigned long long fmask;    // bit i: instruction q + i ends its bag
};

constexpr int kQuadWin = 7;  // load instructions (28 rows) per window: 6, 7 and 8 measured 22.2, 22.0 and
                             // 21.9 us on the multi-hot batch, and 8 spills 8 bytes per lane
// Bytes every buffer resource of the gather covers, 2^31: at least any table it
// takes (under 2^24 rows of 128 bytes, so a last row ends by 2^31) and less
// than the offset of a slot that reads nothing, so that slot is out of range
// and every other is a row of the table.
constexpr int kQuadRange = static_cast<int>(0x80000000u);

// Lane (k, i) works out instruction q + i (the same for all four quarters) and
// the row of it that quarter k loads.
template <int WIN>
__device__ __forceinline__ void quad_prepare(QuadWindow& w, const int* pos, const int* stage,
                                             const char* const* tbase, int incl, int T, int I, int q, int lane) {
  const int k = lane >> 4, i = lane & 15;
  const int x = q + i;
  const bool valid = i < WIN && x < I;
  // x's bag: the number of bags whose instructions all come before x
  int t = 0;
#pragma unroll
  for (int step = 32; step > 0; step >>= 1) {
    const int c = t + step;
    const int e = __shfl(incl, c - 1 < kWave ? c - 1 : kWave - 1, kWave);
    if (c <= T && e <= x) t = c;
  }
  const int ex_raw = __shfl(incl, t > 0 ? t - 1 : 0, kWave);
  bool flush = false;
  uint32_t roff = 0xFFFFFF00u;  // past kQuadRange: the load returns zeros
  if (valid) {
    const int ex = t > 0 ? ex_raw : 0;
    const int end = pos[t + 1];
    const int p = pos[t] + 4 * (x - ex);
    const int c = min(4, end - p);
    flush = k == 0 && p + c == end;
    if (k < c) {
      const int r = stage[p + k];
      if (r >= 0) roff = static_cast<uint32_t>(r) * 128u;
    }
  } else {
    t = 0;
  }
  const uint64_t base = reinterpret_cast<uint64_t>(tbase[t]);
  w.t = t;
  w.roff = roff;
  w.blo = static_cast<uint32_t>(base);
  w.bhi = static_cast<uint32_t>(base >> 32);
  w.fmask = __ballot(flush);
}

// Lane I of each 16-lane row of the wave, to the whole row (DPP row_newbcast).
template <int I>
__device__ __forceinline__ uint32_t quarter_bcast(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x150 + I, 0xF, 0xF, false));
}

// Instructions I.. of a window: instruction I's table base from lane I, each
// quarter's row offset from lane I of the quarter.
template <int I, int WIN>
__device__ __forceinline__ void quad_issue(const QuadWindow& w, uint2 (&v)[WIN], uint32_t sub8) {
  if constexpr (I < WIN) {
    const uint64_t base = bcast64(w.blo, w.bhi, I);
    const uint32_t off = quarter_bcast<I>(w.roff) + sub8;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), 0, kQuadRange, 0x00020000);
    const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kNonTemporal);
    v[I] = make_uint2(x.x, x.y);
    quad_issue<I + 1, WIN>(w, v, sub8);
  }
}

template <int DT, int WIN>
__device__ __forceinline__ void quad_consume(const QuadWindow& w, uint2 (&v)[WIN], float4& acc, float* Z, int LD,
                                             int lane) {
#pragma unroll
  for (int i = 0; i < WIN; ++i) {
    acc.x += decode_lo<DT>(v[i].x);
    acc.y += decode_hi<DT>(v[i].x);
    acc.z += decode_lo<DT>(v[i].y);
    acc.w += decode_hi<DT>(v[i].y);
    if ((w.fmask >> i) & 1ull) {  // uniform: every lane takes part in the exchanges
      float4 s = acc;
      s.x += __shfl_xor(s.x, 16, kWave);
      s.y += __shfl_xor(s.y, 16, kWave);
      s.z += __shfl_xor(s.z, 16, kWave);
      s.w += __shfl_xor(s.w, 16, kWave);
      s.x += __shfl_xor(s.x, 32, kWave);
      s.y += __shfl_xor(s.y, 32, kWave);
      s.z += __shfl_xor(s.z, 32, kWave);
      s.w += __shfl_xor(s.w, 32, kWave);
      const int t = __builtin_amdgcn_readlane(w.t, i);
      if (lane < 16) *reinterpret_cast<float4*>(Z + (1 + t) * LD + lane * 4) = s;
      acc = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// True when a sample of this launch may take gather_quads (uniform).
__device__ __forceinline__ bool quads_fit(const int* trows, int T, int lane) {
  const bool small = lane >= T || static_cast<uint32_t>(trows[lane < T ? lane : 0]) < (1u << 24);
  return T <= kWave && __ballot(!small) == 0ull;
}

template <int DT, int WIN>
__device__ __forceinline__ void gather_quads(const int* pos, const int* stage, const char* const* tbase, int T,
                                             float* Z, int LD, int tid) {
  const int lane = tid & (kWave - 1);
  // instructions per bag (a bag of n rows takes ceil(n / 4)), scanned over the bags
  int incl = lane < T ? (pos[lane + 1] - pos[lane] + 3) >> 2 : 0;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  const int I = rfl(__shfl(incl, T - 1, kWave));
  const uint32_t sub8 = static_cast<uint32_t>(lane & 15) * 8u;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  QuadWindow wa, wb;
  uint2 va[WIN], vb[WIN];
  quad_prepare<WIN>(wa, pos, stage, tbase, incl, T, I, 0, lane);
  quad_issue<0, WIN>(wa, va, sub8);
  for (int q = 0;;) {
    quad_prepare<WIN>(wb, pos, stage, tbase, incl, T, I, q + WIN, lane);
    quad_issue<0, WIN>(wb, vb, sub8);
    quad_consume<DT, WIN>(wa, va, acc, Z, LD, lane);
    q += WIN;
    if (q >= I) break;
    quad_prepare<WIN>(wa, pos, stage, tbase, incl, T, I, q + WIN, lane);
    quad_issue<0, WIN>(wa, va, sub8);
    quad_consume<DT, WIN>(wb, vb, acc, Z, LD, lane);
    q += WIN;
    if (q >= I) break;
  }
#pragma unroll
  for (int j = 0; j < WIN; ++j) {
    touch(va[j]);
    touch(vb[j]);
  }
}

// Logical block of workgroup bid in the row-streaming kernel. The dispatcher
// deals workgroups out round-robin over the 8 XCDs; here each XCD takes runs
// of 16 consecutive logical blocks, interleaved with the other XCDs' runs. The
// samples in flight at any time then form one compact window of the batch
// (their offsets, indices and output lines likely share DRAM pages), while
// neighbouring samples, which share offset and index cache lines, still meet
// in one XCD's L2. On the 64-table capacity batch: 808 us with each XCD on one
// contiguous eighth of the batch, 789-800 us in plain launch order (3.5% more
// bytes fetched), 792-795 us with runs of 16. A ragged last group keeps the
// plain order, so the map is a bijection on [0, n).
__device__ __forceinline__ int run_block(int bid, int n) {
  constexpr int kRun = 16, kSpan = 8 * kRun;
  const int base = bid / kSpan * kSpan;
  if (base + kSpan > n) return bid;
  const int r = bid - base;
  return base + (r % 8) * kRun + r / 8;
}

// Persistent workgroups: each takes a contiguous chunk of samples and runs,
// per step, [gather | prefetch next offsets and e0] -> [carries, scan of the
// next sample] -> [interaction | next sample's index loads in flight] ->
// [output] -> [stage next indices, reset Z]. The round trips of the next
// sample's offsets, e0 and indices overlap this sample's gather and
// interaction.
//
// With G > 1 (short samples) the workgroup is G groups of 512/G threads, each
// with its own LDS region and its own sample in every step, so G samples'
// latency chains overlap; every group runs the same steps and meets the same
// barriers. In a step past the end of the chunk a group repeats the chunk's
// last sample (all loads in bounds) and writes nothing.
template <int DT, int LB, bool MFMA, int G>
__global__ __launch_bounds__(kRowThreads, 6) void fused_rows_kernel(FwdArgs a, RowLayout L, int chunk) {
  constexpr int NT = kRowThreads / G;  // threads of a group
  constexpr int GW = kRowWaves / G;    // waves of a group
  constexpr int CAP = kStageCap / G;   // staged indices of a group's sample
  extern __shared__ __align__(16) char lds[];
  const char** tbase = reinterpret_cast<const char**>(lds + L.off_tbase);
  int* trows = reinterpret_cast<int*>(lds + L.off_trows);
  float* qsb = reinterpret_cast<float*>(lds + L.off_qsb);

  // one step per workgroup (no next sample to fetch during this one) for G = 1;
  // for G > 1 the host may still launch one step per workgroup (multi false)
  constexpr bool kMulti = G > 1;
  const bool multi = kMulti && chunk > G;
  const int T = a.T, D = a.D, LD = L.LD;
  const int F = T + 1;
  const bool self_pairs = (a.layout & DLRM_PAIRS_SELF) != 0;
  const bool with_emb = (a.layout & DLRM_WITH_EMBEDDINGS) != 0;
  const int P = self_pairs ? F * (F + 1) / 2 : F * (F - 1) / 2;
  const int W = (with_emb ? F * D : D) + P;
  const int grp = G == 1 ? 0 : rfl(static_cast<int>(threadIdx.x) / NT);
  const int wave = rfl((static_cast<int>(threadIdx.x) >> 6) % GW);  // wave within the group
  char* gl = lds + L.off_groups + grp * L.group_bytes;
  int* carry_t = reinterpret_cast<int*>(gl + L.off_carry_t);
  int* stage = reinterpret_cast<int*>(gl + L.off_stage);
  uint8_t* sbag = reinterpret_cast<uint8_t*>(gl + L.off_sbag);
  float* carry = reinterpret_cast<float*>(gl + L.off_carry);
  float* outs = reinterpret_cast<float*>(gl + L.off_out);
  float* Z = reinterpret_cast<float*>(gl + L.off_z);

  const int b_begin = run_block(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x)) * chunk;
  const int b_end = min(a.B, b_begin + chunk);
  if (b_begin >= b_end) return;  // whole workgroup
  // this group's sample in the step that starts at sample bs (past the chunk:
  // the chunk's last sample, not written)
  auto sample_of = [&](int bs) { return G == 1 ? bs : min(bs + grp, b_end - 1); };

  // ---- prologue: first sample's bags, positions, indices, e0
  int pb = 0;
  {
    const int tid = static_cast<int>(threadIdx.x) % NT;
    const int b0 = sample_of(b_begin);
    int* beg = reinterpret_cast<int*>(gl + L.off_beg);
    int* pos = reinterpret_cast<int*>(gl + L.off_pos);
    // e0 goes out with the offsets (D <= NT), not after them
    const float e0v = tid < D ? a.e0[static_cast<size_t>(b0) * D + tid] : 0.f;
    if (threadIdx.x < static_cast<unsigned>(T)) {
      tbase[threadIdx.x] = static_cast<const char*>(a.tabs.ptr[threadIdx.x]);
      trows[threadIdx.x] = a.tabs.rows[threadIdx.x];
      if constexpr (DT == DLRM_Q8T) {
        qsb[2 * threadIdx.x] = a.qscale[threadIdx.x];
        qsb[2 * threadIdx.x + 1] = a.qbias[threadIdx.x];
      }
    }
    if (tid < T) {
      publish_bag(a, tid, b0, a.offsets[tid * a.B + b0], a.offsets[tid * a.B + b0 + 1], beg, pos);
      clear_if_empty(pos, tid, Z, LD, D);
    }
    __syncthreads();
    if (tid < D) Z[tid] = e0v;
    if (wave == 0) scan_positions(pos, T, tid);
    __syncthreads();
    int r[kStagePerThread], tb[kStagePerThread];
    load_stage<NT>(a, beg, pos, T, rfl(pos[T]), r, tb, tid);
    write_stage<NT>(a, r, tb, stage, sbag, trows, tid);
    if (tid < GW) carry_t[tid] = -1;
    __syncthreads();
  }

  for (int bs = b_begin; bs < b_end; bs += G) {
    // The thread index is re-derived opaquely each sample so that the compiler
    // recomputes per-thread addresses instead of keeping them live (and
    // spilled) across the whole loop.
    int tid = static_cast<int>(threadIdx.x) % NT;
    asm volatile("" : "+v"(tid));
    const int b = sample_of(bs);
    const bool active = G == 1 || bs + grp < b_end;  // this group writes its sample
    const bool has_next = kMulti && bs + G < b_end;
    int* beg = reinterpret_cast<int*>(gl + L.off_beg + pb * L.pos_stride);
    int* pos = reinterpret_cast<int*>(gl + L.off_pos + pb * L.pos_stride);
    int* nbeg = reinterpret_cast<int*>(gl + L.off_beg + (pb ^ 1) * L.pos_stride);
    int* npos = reinterpret_cast<int*>(gl + L.off_pos + (pb ^ 1) * L.pos_stride);
    const int N = rfl(pos[T]);

    // next sample's bag ranges and e0: loads in flight during the gather. Every
    // thread issues them, clamped in bounds (the last step re-reads its own
    // sample), so that no branch merges their registers and nothing waits for
    // them before the gather is done.
    int nx0 = 0, nx1 = 0;
    float ne0 = 0.f;
    const int bn = has_next ? sample_of(bs + G) : b;
    if constexpr (kMulti) {
      const int tt = tid < T ? tid : T - 1;
      const int td = tid < D ? tid : D - 1;
      nx0 = a.offsets[tt * a.B + bn];
      nx1 = a.offsets[tt * a.B + bn + 1];
      ne0 = a.e0[static_cast<size_t>(bn) * D + td];
    }

    // gather: wave w of the group sums stream positions [p0, p1) in windows of
    // WIN rows. Each lane first works out the address of "its" row of a window
    // and whether a sum ends there; window k+1's loads are issued before window
    // k is summed. Slots past the range read nothing and return zeros, so
    // every window issues the same number of loads.
    {
      const int p0 = static_cast<int>((static_cast<long long>(N) * wave) / GW);
      const int p1 = static_cast<int>((static_cast<long long>(N) * (wave + 1)) / GW);
      if (p0 < p1) {
        float* cw = carry + wave * D;
        int* ctw = carry_t + wave;
        // fp16 rows of 512 bytes in sample groups keep 4 rows per window: 6 made
        // the compiler spill (52-56 bytes per lane), and 4 measured 35.1 against
        // 40.0 us on 26 tables of D = 256 with one index per bag (one sample per
        // workgroup keeps 6: 86.9 against 88.2 us with 20 rows per bag)
        constexpr int WIN = (DT == DLRM_F16 && LB == 8 && G > 1) ? 4 : RowShape<DT, LB>::WIN;
        // 128-byte 16-bit rows with one wave per sample: four rows per load
        constexpr bool kQuads = (DT == DLRM_F16 || DT == DLRM_BF16) && LB == 2 && GW == 1;
        bool done = false;
        if constexpr (kQuads) {
          if (p1 <= CAP && quads_fit(trows, T, tid & (kWave - 1))) {
            gather_quads<DT, kQuadWin>(pos, stage, tbase, T, Z, LD, tid);
            done = true;
          }
        }
        if (!done) {
          if (p1 <= CAP)
            gather_range<DT, LB, false, CAP, WIN>(a, beg, pos, stage, sbag, tbase, trows, T, p0, p1, Z, LD, cw, ctw,
                                                  tid, qsb);
          else
            gather_range<DT, LB, true, CAP, WIN>(a, beg, pos, stage, sbag, tbase, trows, T, p0, p1, Z, LD, cw, ctw,
                                                 tid, qsb);
        }
      }
    }
    // the prefetched values are first used here (the barrier keeps every use,
    // and the wait for them, after the gather)
    if constexpr (kMulti) asm volatile("" : "+v"(nx0), "+v"(nx1), "+v"(ne0));
    bool next_empty = false;
    if (has_next && tid < T) {
      publish_bag(a, tid, bn, nx0, nx1, nbeg, npos);
      next_empty = npos[tid + 1] == 0;
    }
    __syncthreads();

    // bags cut by a range boundary: add the later parts in wave order; scan the next positions
    for (int d = tid; d < D; d += NT) {
      for (int w = 1; w < GW; ++w) {
        const int t = carry_t[w];
        if (t >= 0) Z[(1 + t) * LD + d] += carry[w * D + d];
      }
    }
    if (has_next && wave == GW - 1) scan_positions(npos, T, tid);
    __syncthreads();

    // next sample's index loads go out now; their values are staged after the output
    int r[kStagePerThread], tb[kStagePerThread];
    if (multi) {
      // (issued unconditionally in a multi-step launch, with no positions when
      // there is no next sample: every load stays in bounds and no branch
      // inside the launch's steps merges the registers)
      load_stage<NT>(a, nbeg, npos, T, has_next ? rfl(npos[T]) : 0, r, tb, tid);
    }

    // pooled output (if requested) from the final fp32 Z
    if (a.out_pooled && active) {
      float* op = a.out_pooled + static_cast<size_t>(b) * T * D;
      for (int i = tid; i < T * D; i += NT) {
        const int t = i / D, d = i - t * D;
        op[i] = Z[(1 + t) * LD + d];
      }
    }
    // interaction into the output staging area (which overlays the index
    // stage): [e0 | dots], or only the dots when the Z rows go out as well
    float* dots = with_emb ? outs : outs + D;
    if (!with_emb)
      for (int d = tid; d < D; d += NT) outs[d] = Z[d];
    if constexpr (MFMA && DT == DLRM_F32) {
      // the Gram of every Z row on MFMA with three-way bf16 splits, in 32x32
      // tiles (one for up to 32 Z rows). 26-table batch: 17.7 us per launch
      // against 18.5 us with 16x16 tiles (three tiles on two waves).
      const int nt = (F + 31) / 32;
      const int ntiles = nt * (nt + 1) / 2;
      for (int tile = wave; tile < ntiles; tile += GW) {
        int I, J;
        block_pair(tile, I, J);
        gram_tile32_x6(Z, LD, D, F, I, J, dots, self_pairs, tid & (kWave - 1));
      }
    } else if constexpr (MFMA) {
      // e0 dots in fp32; the Gram of the pooled rows on MFMA, every operand
      // split into bf16 hi + lo in registers as it is read from LDS
      e0_dots<NT>(Z, LD, D, T, dots, tid, self_pairs);
      const int nt = L.Tp / 16;
      const int ntiles = nt * (nt + 1) / 2;
      for (int tile = wave; tile < ntiles; tile += GW) {
        int I, J;
        block_pair(tile, I, J);
        gram_tile16(Z, LD, D, T, I, J, dots, self_pairs, tid & (kWave - 1));
      }
    } else {  // fp32 dots, one 4x4 block of pairs per 16 lanes
      const int nb = (T + 1 + 3) >> 2;
      for (int u = tid >> 4; u < nb * (nb + 1) / 2; u += NT / 16) {
        int bi, bj;
        block_pair(u, bi, bj);
        dots_block16<true>(Z, T + 1, D, LD, bi, bj, tid & 15, dots, self_pairs);
      }
    }
    __syncthreads();
    // the next sample's index loads have had the whole interaction to land:
    // take them now, before the output stores are queued behind them
    if (multi) {
#pragma unroll
      for (int k = 0; k < kStagePerThread; ++k) asm volatile("" : "+v"(r[k]));
    }
    if (active) {
      const __amdgpu_buffer_rsrc_t ro =
          row_rsrc(reinterpret_cast<uint64_t>(a.out_inter + static_cast<size_t>(b) * W), W * 4);
      if (with_emb) {  // [Z_0 | Z_1 .. Z_T | dots]
        for (int i = tid; i < F * D; i += NT) {
          const int f = i / D, d = i - f * D;
          store_out(ro, i, Z[f * LD + d]);
        }
        for (int i = tid; i < P; i += NT) store_out(ro, F * D + i, outs[i]);
      } else {
        for (int i = tid; i < W; i += NT) store_out(ro, i, outs[i]);
      }
    }
    __syncthreads();

    // stage the next sample: indices, cleared Z with its e0, no carries
    if (has_next) {
      if (multi) write_stage<NT>(a, r, tb, stage, sbag, trows, tid);
      if (next_empty) {
        float* z = Z + (1 + tid) * LD;
        for (int d = 0; d < D; d += 4) *reinterpret_cast<float4*>(z + d) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (tid < GW) carry_t[tid] = -1;
      if (tid < D) Z[tid] = ne0;
      __syncthreads();
    }
    pb ^= 1;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int fwd_supported_row_bytes(int D, int dtype) {
  // bytes of one row's values: D codes of one byte (table-wise 8-bit), D / 2 (4-bit)
  const long rb = dtype == DLRM_Q4 ? D / 2
                  : static_cast<long>(D) * (dtype == DLRM_F32 ? 4 : dtype == DLRM_Q8T ? 1 : 2);
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

// Row-streaming fused kernel: rows of 128..1024 bytes (16-bit storage) or
// 256..1024 bytes (fp32); MFMA interaction for 16-bit storage with T >= 24.
static bool use_row_kernel(int D, int dtype) {
  const int rb = fwd_supported_row_bytes(D, dtype);
  if (dtype == DLRM_Q4 || dtype == DLRM_Q8T) return rb >= 64 && rb <= 512;  // the only kernel for quantized rows
  return dtype == DLRM_F32 ? (rb >= 256 && rb <= 1024) : (rb >= 128 && rb <= 1024);
}
// MFMA only where the per-sample Gram is a real dense contraction (F >= 25):
// a bf16 hi + lo split of the pooled rows for 16-bit and quantized tables, a
// three-way split of every Z row for fp32 tables.
static bool use_mfma(int T, int D, int /*dtype*/) { return T >= 24 && D % 16 == 0; }
// Z needs whole 32-row tiles only for the two-way split (its tiles do not
// clamp their rows).
static bool padded_z(int T, int D, int dtype) { return dtype != DLRM_F32 && use_mfma(T, D, dtype); }

size_t fwd_lds_bytes(int T, int D, int dtype) {
  if (use_row_kernel(D, dtype)) return static_cast<size_t>(make_row_layout(T, D, padded_z(T, D, dtype)).bytes);
  const Tile tl = make_tile(T, D, 1);
  return tl.z_floats() * 4 + static_cast<size_t>(T) * 2 * 4;
}

// Persistent grid: as many 512-thread workgroups as the device keeps resident
// at this LDS size, each with a contiguous chunk of samples.
template <class K>
static int resident_blocks(K kernel, size_t lds) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kRowThreads, lds) != hipSuccess) return 0;
  return cus * (per_cu > 0 ? per_cu : 1);
}

constexpr int kLongSampleRows = 512;  // average rows per sample from which a workgroup takes one sample

// Sample groups per workgroup for short samples: as many as keep a group's
// threads covering the bags and e0 (G * max(T, D) <= 512), the staged indices
// covering a typical sample with room to spare, the LDS within one CU's, and
// at least 64 workgroups of G samples.
static int pick_groups(const FwdArgs& a, bool mfma) {
  if (a.nnz >= static_cast<int64_t>(kLongSampleRows) * a.B) return 1;
  const int64_t avg = a.nnz / a.B;  // rows per sample
  const int wide = a.T > a.D ? a.T : a.D;
  for (int G = 8; G > 1; G /= 2) {
    if (G * wide > kRowThreads) continue;
    if (avg * 3 / 2 > kStageCap / G) continue;
    if (static_cast<size_t>(make_row_layout(a.T, a.D, mfma, G).bytes) > kMaxLds) continue;
    if (a.B < G * 64) continue;
    return G;
  }
  return 1;
}

template <int DT, int LB, bool MFMA, int G>
static hipError_t launch_rows_g(const FwdArgs& a, hipStream_t st) {
  const RowLayout L = make_row_layout(a.T, a.D, MFMA && DT != DLRM_F32, G);
  auto kernel = fused_rows_kernel<DT, LB, MFMA, G>;
  // Short samples: two steps per workgroup, the second step's offsets, e0 and
  // indices fetched while the first is gathered. Long samples (hundreds of
  // rows): one per workgroup, which keeps the end of the launch short (the
  // hardware dispatcher hands the many short-lived workgroups to free slots).
  const bool long_samples = a.nnz >= static_cast<int64_t>(kLongSampleRows) * a.B;
  const int steps =
      (G > 1 && !long_samples && a.B >= 2 * G * resident_blocks(kernel, static_cast<size_t>(L.bytes))) ? 2 : 1;
  const int chunk = G * steps;
  const int grid = (a.B + chunk - 1) / chunk;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kRowThreads), L.bytes, st, a, L, chunk);
  return hipGetLastError();
}

template <int DT, int LB, bool MFMA>
static hipError_t launch_rows_m(const FwdArgs& a, hipStream_t st) {
  switch (pick_groups(a, MFMA && DT != DLRM_F32)) {
    case 8: return launch_rows_g<DT, LB, MFMA, 8>(a, st);
    case 4: return launch_rows_g<DT, LB, MFMA, 4>(a, st);
    case 2: return launch_rows_g<DT, LB, MFMA, 2>(a, st);
    default: return launch_rows_g<DT, LB, MFMA, 1>(a, st);
  }
}

template <int DT, int LB>
static hipError_t launch_rows(const FwdArgs& a, hipStream_t st) {
  const bool mfma = use_mfma(a.T, a.D, DT);
  if (static_cast<size_t>(make_row_layout(a.T, a.D, padded_z(a.T, a.D, DT)).bytes) > kMaxLds)
    return hipErrorInvalidValue;
  if (mfma) return launch_rows_m<DT, LB, true>(a, st);
  return launch_rows_m<DT, LB, false>(a, st);
}

template <int DT, int LPR>
static hipError_t launch_fwd_float(const FwdArgs& a, hipStream_t st) {
  if (a.out_inter && use_row_kernel(a.D, DT)) {
    constexpr int LB = LPR * 16 / kWave;  // bytes per lane when one wave reads one row
    if constexpr (LB == 2 && DT != DLRM_F32) return launch_rows<DT, 2>(a, st);
    else if constexpr (LB == 4) return launch_rows<DT, 4>(a, st);
    else if constexpr (LB == 8) return launch_rows<DT, 8>(a, st);
    else if constexpr (LB == 16) return launch_rows<DT, 16>(a, st);
    else return hipErrorInvalidValue;
  }
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

template <int DT, int LPR>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  if constexpr (DT == DLRM_Q4 || DT == DLRM_Q8T) {  // quantized rows: row-streaming fused kernel only
    constexpr int LB = LPR * 16 / kWave;  // code bytes per lane
    if (!a.out_inter) return hipErrorInvalidValue;
    if constexpr (DT == DLRM_Q4 && (LB == 1 || LB == 2 || LB == 4)) return launch_rows<DT, LB>(a, st);
    else if constexpr (DT == DLRM_Q8T && (LB == 2 || LB == 4 || LB == 8)) return launch_rows<DT, LB>(a, st);
    else return hipErrorInvalidValue;
  } else {
    return launch_fwd_float<DT, LPR>(a, st);
  }
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
    case DLRM_Q4: return launch_fwd_dt<DLRM_Q4>(a, st);
    case DLRM_Q8T: return launch_fwd_dt<DLRM_Q8T>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_interact(int T, int B, int D, int layout, const float* e0, const float* pooled, float* out,
                           hipStream_t st) {
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
  hipLaunchKernelGGL(interact_kernel, dim3(grid), dim3(kThreads), lds, st, T, B, D, e0, pooled, out, S, layout);
  return hipGetLastError();
}

}  // namespace dlrm
